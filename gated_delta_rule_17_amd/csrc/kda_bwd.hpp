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
//                 beta scaling), T, W and W^T, U, Kr and Kr^T, and the two
//                 products with dO that the reverse carry would otherwise
//                 repeat each step, Ut = Aqk^T dO and P = (scale Q e^G)^T dO,
//                 into per-chunk float32 records.
//   2. bwd_states one launch, two roles: workgroups of the first half carry
//                 the state forward through the chunks (storing the state
//                 entering each chunk and E), those of the second half carry
//                 the state gradient backward,
//                   dE = Ut + Kr dH' ;
//                   dH = Diag(e^{G_last}) dH' + P - W^T dE,
//                 storing dH' and dE per chunk.  Each workgroup owns one
//                 16-column tile of the value dimension of one head.  For
//                 bf16 inputs (bwd_states_mc) W, W^T, Kr and Kr^T come as bf16
//                 pairs in matrix-core fragment order and the products run on
//                 the bf16 matrix cores.
//   3. bwd_grad   one workgroup per chunk, one wave per 16 key channels:
//                 dUt = T^T dE, dv = beta dUt, the products with the chunk
//                 state and its gradient, dA = -(strict lower dUt E^T),
//                 dAqk = lower dO E^T, then dq, dk, dbeta and the gate
//                 gradient (suffix sums of dG inside the chunk).
//   4. bwd_group_sum (grouped value heads only) adds the query/key gradients
//                 of the value heads that share a query/key head.
//
// Products run on v_mfma_f32_16x16x4_f32 with float32 operands from LDS
// (operand convention, lane l, r = l % 16, g = l / 16: A[r][g], B[g][r];
// accumulator element i is D[4g + i][r]), except the products over the value
// dimension in bwd_grad and, for bf16 inputs, the products with T, Aqk and
// scale Q e^G in bwd_prep: those take v_mfma_f32_16x16x32_bf16 over bf16
// parts (hi + mid + lo) of their float32 operands, which keeps them good to
// about 2^-24 of each operand; and, for bf16 inputs, the state passes, over
// hi + lo pairs (about 2^-16).
//
// Decays inside a chunk come from differences of G.  Products that sum
// over the tokens of a chunk with a decay between the two tokens are split
// at a reference row per 16-row output block: the first row of the block for
// sums over earlier tokens, the last row for sums over later ones.  Every
// factor is then either at most 1 or spans at most 15 tokens.  A key channel
// whose decay across one block exceeds e^-kBlockRange (a hard forget) would
// overflow the factor that spans the block; that (block, channel) is left
// out of the block's own product and its in-block terms are summed exactly,
// exp(G_i - G_j) <= 1 pair by pair, in a fixed order.
#pragma once

#include <atomic>
#include <type_traits>

#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace bwd {

// Per-chunk float32 records in the workspace; record r = unit * NC + chunk,
// unit = b * H + h (dense batch), or r = h * Gmax + g for chunk slot g of a
// packed batch (the chunks of one sequence are consecutive slots).  Rows of a ragged last chunk beyond its length are zero
// (G repeats its last valid row).
// W, WT, Kr and KrT of bf16 inputs (prep_split) hold instead the bf16 pairs
// of store_mc in the same bytes: fragments of [C][DK] (W, Kr) and of [DK][C]
// (WT, KrT), hi plane then lo plane.
struct Records {
    float* G;    // [C][DK]  inclusive prefix of the log gates
    float* W;    // [C][DK]
    float* WT;   // [DK][C]  W transposed
    float* Kr;   // [C][DK]  K e^{G_last - G}
    float* KrT;  // [DK][C]  Kr transposed
    float* U;    // [DV][C]  U transposed
    float* Ut;   // [DV][C]  (Aqk^T dO) transposed
    float* P;    // [DV][DK] ((scale Q e^G)^T dO) transposed
    float* Tm;   // [C][C]   (I + A)^-1
    float* Ap;   // [C][C]   A before the beta scaling (strict lower)
    float* Hs;   // [DV][DK] state entering the chunk, transposed (= S)
    float* E;    // [DV][C]  pseudo-values, transposed
    float* dH;   // [DV][DK] gradient of the state leaving the chunk, transposed
    float* dE;   // [DV][C]  transposed
    size_t rs;   // floats from one record to the next: the fields of one
                 // (sequence, head, chunk) lie together in one block
};

struct Args {
    const void* q; const void* k; const void* v; const void* dO;
    const float* g; const float* beta; const float* h0; const float* dhT;
    void* dq; void* dk; void* dv;
    float* dg; float* dbeta; float* dh0;
    float* dqp; float* dkp;   // grouped heads: float partials per value head, else null
    Records r;
    int B, T, H, Hq, NC, mode;
    // packed batch: chunk table (first token, length) of Gmax slots, sequence
    // table (first token, length, first slot, 0) of N sequences; B = 1 and T
    // the packed token count.  Null for a dense batch.
    const int2* ctab;
    const int4* stab;
    int N, Gmax;
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

// A key channel whose log gates fall by more than this across one 16-row block
// (block, channel "flagged") is left out of that block's factored products,
// whose key side grows to exp(G at the block's first row - G at its last row);
// the block's terms of that channel are taken exactly, exp(G_i - G_j) <= 1 for
// each pair, on the vector units instead.
constexpr float kBlockRange = 80.f;

// Workgroup barrier that orders LDS only: LDS writes before it are visible to
// LDS reads after it, while global loads and stores stay in flight.
// __syncthreads() also waits for every outstanding global access, and since
// the vector-memory counter retires in order, a record store issued after a
// prefetch then holds the barrier until the prefetch has landed.  Every
// exchange between the waves of these kernels goes through LDS.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Orders this wave's LDS writes before its later LDS reads, for lanes of one
// wave that exchange values through a buffer of their own (no other wave
// takes part, so no workgroup barrier is needed).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Inclusive prefix sum over the 16 lanes of a DPP row (row_shr 1, 2, 4, 8;
// lanes shifted in from outside the row contribute zero): lane 15 of the row
// ends with the row's total.  Pure VALU, no LDS round trip.
__device__ __forceinline__ float row16_scan(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xf, 0xf, false));
    return x;
}

// Loads of a chunk's rows are issued unconditionally from a clamped row
// (every chunk has at least one row) and zeroed past the end afterwards: a
// load under a per-row branch is waited for at the branch join, which
// serialises the loads of a thread.
__device__ __forceinline__ int clamp_row(int i, int L) { return i < L ? i : L - 1; }
__device__ __forceinline__ float keep(float x, int i, int L) { return i < L ? x : 0.f; }

// The gate of row i as base[i * stride], branch-free over the three modes
// (the ungated mode reads beta and scales it by zero).
struct GatePtr {
    const float* base;
    size_t stride;
    float mul;
};
__device__ __forceinline__ GatePtr gate_ptr(const Args& a, int b, int t0, int h, int c, int DK) {
    const size_t row0 = ((size_t)b * a.T + t0) * a.H + h;
    if (a.mode == KDA_GATE_CHANNEL) return {a.g + row0 * DK + c, (size_t)a.H * DK, 1.f};
    if (a.mode == KDA_GATE_SCALAR) return {a.g + row0, (size_t)a.H, 1.f};
    return {a.beta + row0, (size_t)a.H, 0.f};
}

// The chunk of a per-chunk workgroup: batch entry, value head, first token
// and length (0 for an empty slot of a packed batch).
struct ChunkLoc {
    int b, h, t0, L;
};
template <int C>
__device__ __forceinline__ ChunkLoc locate_chunk(const Args& a, int rec) {
    ChunkLoc l;
    if (a.ctab) {
        l.b = 0;
        l.h = rec / a.Gmax;
        const int2 e = a.ctab[rec % a.Gmax];
        l.t0 = e.x;
        l.L = e.y;
    } else {
        const int u = rec / a.NC, ch = rec % a.NC;
        l.b = u / a.H;
        l.h = u % a.H;
        l.t0 = ch * C;
        l.L = min(C, a.T - l.t0);
    }
    return l;
}

// Compute units of the current device, queried once per device (256 if the
// query fails; its error is then cleared so that no later launch check sees it).
inline int device_cus()
{
    constexpr int MAXDEV = 64;
    static std::atomic<int> cache[MAXDEV];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        dev = 0;
    }
    const int slot = dev < MAXDEV ? dev : MAXDEV - 1;
    int n = cache[slot].load(std::memory_order_relaxed);
    if (n > 0 && dev < MAXDEV) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) {
        (void)hipGetLastError();
        n = 256;
    }
    if (dev < MAXDEV) cache[slot].store(n, std::memory_order_relaxed);
    return n;
}

// Index of the n-th lower block tile (I, J), J <= I, of an NB x NB grid.
__device__ __forceinline__ void lower_tile(int n, int& I, int& J) {
    I = 0;
    while (n > I) { n -= I + 1; ++I; }
    J = n;
}

// ---- products over bf16 parts of float32 operands ---------------------------
// x = hi + mid + lo in bf16 parts (each the nearest bf16 to what the
// previous parts leave; the differences are exact in float32), good to
// about 2^-24 of x.
__device__ __forceinline__ void split3(float x, uint16_t& hi, uint16_t& mid, uint16_t& lo) {
    hi = f32_to_bf16(x);
    const float r = x - bf16_to_f32(hi);
    mid = f32_to_bf16(r);
    lo = f32_to_bf16(r - bf16_to_f32(mid));
}

// The same for a pair of values, each part packed two to a word (value 0 in
// the low half): one conversion instruction per part for both values, with
// the rounding of f32_to_bf16.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_pk(float x0, float x1) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){x0, x1}, bf16x2_t));
}
__device__ __forceinline__ void split3x2(float x0, float x1, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
    hi = cvt_pk(x0, x1);
    const float r0 = x0 - __uint_as_float(hi << 16), r1 = x1 - __uint_as_float(hi & 0xffff0000u);
    mid = cvt_pk(r0, r1);
    lo = cvt_pk(r0 - __uint_as_float(mid << 16), r1 - __uint_as_float(mid & 0xffff0000u));
}

// Planes of bf16 rows (pw 32-bit words per row); a fragment is the 8
// consecutive values at columns 8 q4 .. 8 q4 + 7 of one row, which is the
// operand of lane (r, q4) of v_mfma_f32_16x16x32_bf16 (A[r][8g..8g+7] and
// B[8g..8g+7][r]; the accumulator is laid out as for the float32
// instruction).  The three parts of a split operand sit in three planes ps
// words apart.
struct F3 { u16x8 h, m, l; };
__device__ __forceinline__ u16x8 pfrag(const uint32_t* plane, int pw, int row, int q4) {
    return *reinterpret_cast<const u16x8*>(plane + row * pw + 4 * q4);
}
__device__ __forceinline__ F3 pfrag3(const uint32_t* plane, int ps, int pw, int row, int q4) {
    return F3{pfrag(plane, pw, row, q4), pfrag(plane + ps, pw, row, q4), pfrag(plane + 2 * ps, pw, row, q4)};
}
__device__ __forceinline__ f32x4 mmb(const u16x8& x, const u16x8& y, f32x4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x), __builtin_bit_cast(bf16x8, y),
                                                   acc, 0, 0, 0);
}
// both operands split: hh + hm + mh + hl + lh + mm (smallest terms first)
__device__ __forceinline__ f32x4 mm6(const F3& x, const F3& y, f32x4 acc) {
    acc = mmb(x.m, y.m, acc);
    acc = mmb(x.l, y.h, acc);
    acc = mmb(x.h, y.l, acc);
    acc = mmb(x.m, y.h, acc);
    acc = mmb(x.h, y.m, acc);
    return mmb(x.h, y.h, acc);
}
// one operand exact in bf16
__device__ __forceinline__ f32x4 mm3a(const u16x8& x, const F3& y, f32x4 acc) {
    acc = mmb(x, y.l, acc);
    acc = mmb(x, y.m, acc);
    return mmb(x, y.h, acc);
}
__device__ __forceinline__ f32x4 mm3b(const F3& x, const u16x8& y, f32x4 acc) {
    acc = mmb(x.l, y, acc);
    acc = mmb(x.m, y, acc);
    return mmb(x.h, y, acc);
}
// eight consecutive values of a row into the three part planes
__device__ __forceinline__ void put3x8(uint32_t* plane, int ps, int off, const float* x) {
    uint32_t h[4], m[4], l[4];
#pragma unroll
    for (int z = 0; z < 4; ++z) split3x2(x[2 * z], x[2 * z + 1], h[z], m[z], l[z]);
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    *reinterpret_cast<u32x4_t*>(plane + off) = (u32x4_t){h[0], h[1], h[2], h[3]};
    *reinterpret_cast<u32x4_t*>(plane + ps + off) = (u32x4_t){m[0], m[1], m[2], m[3]};
    *reinterpret_cast<u32x4_t*>(plane + 2 * ps + off) = (u32x4_t){l[0], l[1], l[2], l[3]};
}
// eight values exact in bf16 into one plane
__device__ __forceinline__ void put1x8(uint32_t* plane, int off, const float* x) {
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    *reinterpret_cast<u32x4_t*>(plane + off) =
        (u32x4_t){cvt_pk(x[0], x[1]), cvt_pk(x[2], x[3]), cvt_pk(x[4], x[5]), cvt_pk(x[6], x[7])};
}

// ---- 16-byte loads through a buffer resource ----------------------------------
// The base address sits in scalar registers (one resource per record) and each
// lane supplies a 32-bit byte offset, so a loop that walks the records keeps no
// 64-bit vector addresses; soff is a constant added on top.
// A resource of zero length returns zeros without a memory access.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t record_rsrc(const void* base, int bytes = 0x7fffffff) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
template <typename V>
__device__ __forceinline__ V bload(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
    return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ float bload1(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}

// Value of lane J of this lane's 16-lane row (DPP row broadcast).
template <int J>
__device__ __forceinline__ float row_bcast(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + J, 0xf, 0xf, false));
}

// ---- operands of the matrix-core state passes (bf16 inputs) -----------------
// An operand of logical shape [rows][K] (K = 32 KSn) is stored as its 16 x 32
// fragments (row tile, k step), each as 64 lanes x 8 values, so that one
// wave's fragment load is 1 KiB of contiguous memory.  Lane (r, g) of
// fragment (rt, ks) holds row 16 rt + r; its value e is the one at
// k = 32 ks + 16 (e / 4) + 4 g + e % 4.  A lane thus holds two runs of four
// consecutive k, which is how the 16 x 16 accumulators of two adjacent tiles
// hold a column: the producer's accumulators are a fragment as they stand.
// The contraction is the same for any order of k as long as both operands
// use it; the state and E staged in LDS for the other side follow it too.
// The values are float32 stored as bf16 pairs, hi = bf16(x) and
// lo = bf16(x - hi), in two planes `plane` elements apart.
__device__ __forceinline__ int mc_pos(int k) {   // position of k within its 32-wide step
    return 8 * ((k >> 2) & 3) + 4 * ((k >> 4) & 1) + (k & 3);
}
__device__ __forceinline__ void store_mc(uint16_t* base, int plane, int idx, f32x4 x0, f32x4 x1) {
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    uint32_t h[4], l[4];
#pragma unroll
    for (int z = 0; z < 2; ++z) {
        const f32x4 x = z ? x1 : x0;
        h[2 * z] = cvt_pk(x[0], x[1]);
        h[2 * z + 1] = cvt_pk(x[2], x[3]);
        l[2 * z] = cvt_pk(x[0] - __uint_as_float(h[2 * z] << 16), x[1] - __uint_as_float(h[2 * z] & 0xffff0000u));
        l[2 * z + 1] = cvt_pk(x[2] - __uint_as_float(h[2 * z + 1] << 16),
                              x[3] - __uint_as_float(h[2 * z + 1] & 0xffff0000u));
    }
    *reinterpret_cast<u32x4_t*>(base + idx) = (u32x4_t){h[0], h[1], h[2], h[3]};
    *reinterpret_cast<u32x4_t*>(base + plane + idx) = (u32x4_t){l[0], l[1], l[2], l[3]};
}

// ---------------------------------------------------------------------------
// 1. per-chunk preparation
// ---------------------------------------------------------------------------
template <int C, int DK, int DV>
constexpr int prep_threads() { return (C * DK >= 512 && C * DV >= 512) ? 512 : 256; }

// bf16 inputs: the products with T, Aqk and (scale Q e^G) run on bf16 matrix
// cores over split operands (v and dO are exact in bf16), where the chunk is
// a multiple of the 32-wide step and each thread's rows come in whole 8-row
// groups
template <int C, int DK, int DV, typename IO>
constexpr bool prep_split()
{
    constexpr int NT = prep_threads<C, DK, DV>();
    return std::is_same<IO, bf16_t>::value && C % 32 == 0 && (C * DK / NT) % 8 == 0 &&
           (C * DV / NT) % 8 == 0;
}

// SPL: the split path, whose float32 staging rows hold key channels only
template <int C, int DK, int DV, bool SPL>
struct PrepLds {
    static constexpr int NB = C / 16;
    static constexpr int DM = SPL || DK > DV ? DK : DV;
    static constexpr int LS = DM + 2, LK = DK + 2, LC = C + 2, LQ = C + 16;
    static constexpr int LO = DV + 16, LG = DK + 16;
    // phase 1: couplings, inverse, W, U
    static constexpr int oS = 0, oAk = oS + C * LS, oAq = oAk + 16 * LK, oAp = oAq + 16 * LK,
                         oT = oAp + C * LC, P1_END = oT + C * LC;
    // phase 2: Aqk^T dO and (scale Q e^G)^T dO, over the phase-1 buffers
    static constexpr int odO = 0, oQg = odO + C * LO, P2_END = oQg + C * LG;
    // Aqk lives through both phases
    static constexpr int oAqk = P1_END > P2_END ? P1_END : P2_END;
    static constexpr int SIZE = oAqk + C * LQ;
    // split path (bf16 inputs): bf16 planes whose rows hold C + 8 values along
    // the chunk (PW words per row).  (K e^G)^T and V^T overlay phase 1 once T
    // has been read; T Diag(beta) sits past phase 1; (scale Q e^G)^T and dO^T
    // overlay both; Aqk^T lives past everything from the coupling phase on.
    static constexpr int PW = (C + 8) / 2;
    static constexpr int xKG = 0, xVT = xKG + 3 * DK * PW, X2_END = xVT + DV * PW;
    static constexpr int xTB = P1_END > X2_END ? P1_END : X2_END, XT_END = xTB + 3 * C * PW;
    static constexpr int yQG = 0, ydO = yQG + 3 * DK * PW, Y_END = ydO + DV * PW;
    static constexpr int oAqkP = XT_END > Y_END ? XT_END : Y_END;
    static constexpr int SIZE_S = oAqkP + 3 * C * PW;
};

template <int C, int DK, int DV, typename IO>
__global__ void __launch_bounds__((prep_threads<C, DK, DV>())) bwd_prep(Args a)
{
    constexpr bool SPLIT = prep_split<C, DK, DV, IO>();
    using S = PrepLds<C, DK, DV, SPLIT>;
    constexpr int NB = S::NB, LS = S::LS, LK = S::LK, LC = S::LC, LQ = S::LQ, LO = S::LO,
                  LG = S::LG;
    constexpr int NT = prep_threads<C, DK, DV>(), NW = NT / 64;
    constexpr int TPC = NT / DK, RPT = C / TPC;    // threads per key channel, rows per thread
    constexpr int TPV = NT / DV, RPV = C / TPV;    // the same for value channels
    constexpr int PW = S::PW;
    __shared__ __align__(16) float smem[SPLIT ? S::SIZE_S : S::SIZE];
    __shared__ float sGref[NB + 1][DK];             // G at rows 16 I and at the last row
    __shared__ float sSeg[TPC][DK];
    __shared__ float sBeta[C];
    constexpr int FW = (DK + 31) / 32;
    __shared__ uint32_t sFlag[NB][FW];              // flagged (block, channel) pairs
    __shared__ float sX[3][16][17];                 // G, k, scale q of 16 flagged channels x 16 rows
    __shared__ float sEx[2][16][17];                // exact diagonal-block terms: Ap, Aqk
    float* const sS = smem + S::oS;
    float* const sAk = smem + S::oAk;
    float* const sAq = smem + S::oAq;
    float* const sAp = smem + S::oAp;
    float* const sT = smem + S::oT;
    float* const sdO = smem + S::odO;
    float* const sQg = smem + S::oQg;
    float* const sAqk = smem + S::oAqk;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r16 = lane & 15, q4 = lane >> 4;
    const int rec = blockIdx.x;
    const ChunkLoc loc = locate_chunk<C>(a, rec);
    if (loc.L <= 0) return;                  // empty slot of a packed batch
    const int b = loc.b, h = loc.h, hq = h / (a.H / a.Hq);
    const int t0 = loc.t0;
    const int L = loc.L;
    const IO* q = (const IO*)a.q;
    const IO* k = (const IO*)a.k;
    const IO* v = (const IO*)a.v;
    const IO* dO = (const IO*)a.dO;
    const size_t R = (size_t)rec;

    // this thread's elements: key channel c, rows r0 .. r0 + RPT - 1
    const int c = tid % DK, seg = tid / DK, r0 = seg * RPT;
    float kr[RPT], qr[RPT], Gr[RPT];
    {
        // the gates first: loads complete in order, and the scan below needs
        // only them
        const GatePtr gp = gate_ptr(a, b, t0, h, c, DK);
#pragma unroll
        for (int m = 0; m < RPT; ++m) Gr[m] = gp.base[clamp_row(r0 + m, L) * gp.stride] * gp.mul;
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const size_t o = tok_qk(a, b, t0 + clamp_row(r0 + m, L), hq) * DK + c;
            kr[m] = io<IO>::load(k + o);
            qr[m] = io<IO>::load(q + o);
        }
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            kr[m] = keep(kr[m], r0 + m, L);
            qr[m] = keep(qr[m], r0 + m, L);
            Gr[m] = keep(Gr[m], r0 + m, L);
        }
    }
    // G: inclusive prefix per channel (segment scans, then segment offsets)
#pragma unroll
    for (int m = 1; m < RPT; ++m) Gr[m] += Gr[m - 1];
    sSeg[seg][c] = Gr[RPT - 1];
    for (int i = tid; i < C; i += NT) sBeta[i] = i < L ? a.beta[tok_v(a, b, t0 + i, h)] : 0.f;
    for (int i = tid; i < NB * FW; i += NT) sFlag[i / FW][i % FW] = 0u;
    lds_barrier();
    {
        float off = 0.f;
        for (int s2 = 0; s2 < seg; ++s2) off += sSeg[s2][c];
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            Gr[m] += off;
            const int i = r0 + m;
            a.r.G[R * a.r.rs + i * DK + c] = Gr[m];
            if (i % 16 == 0) sGref[i / 16][c] = Gr[m];
            if (i == C - 1) sGref[NB][c] = Gr[m];
        }
    }
    lds_barrier();
    // flagged (block, channel) pairs: the thread holding a block's last row
    // compares it with the block's first row (bitwise OR is order-free)
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = r0 + m;
        if (i % 16 == 15 && sGref[i / 16][c] - Gr[m] > kBlockRange)
            atomicOr(&sFlag[i / 16][c >> 5], 1u << (c & 31));
    }
    lds_barrier();

    // couplings, one 16-row block I at a time with reference row 16 I:
    // Ap = strict lower K Gamma K^T (before beta), Aqk = inclusive lower Q~ Gamma K^T
    if constexpr (SPLIT) {
        // Aqk^T blocks (rows 16 (I + 1) .., columns 16 I ..) above the
        // diagonal are read by the 32-wide steps of the Ut products: zero
        uint32_t* pAq = reinterpret_cast<uint32_t*>(smem + S::oAqkP);
        for (int e = tid; e < 3 * (NB - 1) * 32; e += NT) {
            const int part = e / ((NB - 1) * 32), r = e % ((NB - 1) * 32), I = r / 32;
            const int row = 16 * (I + 1) + (r % 32) / 2, col = 16 * I + 8 * (r % 2);
            *reinterpret_cast<u16x8*>(pAq + part * C * PW + row * PW + col / 2) = (u16x8){0, 0, 0, 0, 0, 0, 0, 0};
        }
    }
    // v and dO rows of this thread's value channel for U, Ut and P, requested
    // here so that they arrive during the coupling phase
    const int cv = tid % DV, r0v = (tid / DV) * RPV;
    float vv[RPV], dv_[RPV];
#pragma unroll
    for (int m = 0; m < RPV; ++m) {
        const size_t o = tok_v(a, b, t0 + clamp_row(r0v + m, L), h) * DV + cv;
        vv[m] = io<IO>::load(v + o);
        dv_[m] = io<IO>::load(dO + o);
    }

    // (a thread's RPT <= 16 rows lie in one 16-row block, Ib, so the row
    // conditions are uniform per thread and the reference is read once)
    static_assert(RPT <= 16 && 16 % RPT == 0, "a thread's rows within one block");
    const int Ib = r0 / 16;
    for (int I = 0; I < NB; ++I) {
        const float gref = sGref[I][c];
        uint32_t anyw = 0;
#pragma unroll
        for (int f = 0; f < FW; ++f) anyw |= sFlag[I][f];
        const bool anyI = anyw != 0;                  // uniform over the workgroup
        if (anyI) {
            // exact terms of the flagged channels inside block I: thread t < 256
            // owns entry (i, j) = (16 I + t / 16, 16 I + t % 16) and adds the
            // channels in ascending order, 16 at a time through sX
            float ea = 0.f, eq = 0.f;
            const int ii = (tid >> 4) & 15, jj = tid & 15;
            for (int cb = 0; cb < DK; cb += 16) {
                const uint32_t bm = (sFlag[I][cb >> 5] >> (cb & 31)) & 0xffffu;
                if (!bm) continue;                    // uniform
                if (Ib == I && c >= cb && c < cb + 16 && ((bm >> (c - cb)) & 1u)) {
#pragma unroll
                    for (int m = 0; m < RPT; ++m) {
                        const int row = r0 + m - 16 * I;
                        sX[0][c - cb][row] = Gr[m];
                        sX[1][c - cb][row] = kr[m];
                        sX[2][c - cb][row] = a.scale * qr[m];
                    }
                }
                lds_barrier();
                if (tid < 256 && jj <= ii) {
                    for (uint32_t mm = bm; mm; mm &= mm - 1) {
                        const int cc = __builtin_ctz(mm);
                        const float kj = sX[1][cc][jj] * ex(sX[0][cc][ii] - sX[0][cc][jj]);
                        if (jj < ii) ea += sX[1][cc][ii] * kj;
                        eq += sX[2][cc][ii] * kj;
                    }
                }
                lds_barrier();
            }
            if (tid < 256) {
                sEx[0][ii][jj] = ea;
                sEx[1][ii][jj] = eq;
            }
        }
        // a flagged channel's key side is left out of the diagonal block
        const bool flc = (sFlag[I][c >> 5] >> (c & 31)) & 1u;
        if (Ib <= I) {
#pragma unroll
            for (int m = 0; m < RPT; ++m)
                sS[(r0 + m) * LS + c] = (Ib == I && flc) ? 0.f : kr[m] * ex(gref - Gr[m]);
        }
        if (Ib == I) {
#pragma unroll
            for (int m = 0; m < RPT; ++m) {
                const int jl = r0 + m - 16 * I;
                const float f = ex(Gr[m] - gref);
                sAk[jl * LK + c] = kr[m] * f;
                sAq[jl * LK + c] = a.scale * qr[m] * f;
            }
        }
        lds_barrier();
        for (int job = w; job < 2 * (I + 1); job += NW) {
            const int which = job & 1, J = job >> 1;
            const float* A = which ? sAq : sAk;
            f32x4 acc = zero4(), acc2 = zero4();   // two independent chains
#pragma unroll 4
            for (int kk = 0; kk < DK; kk += 8) {
                acc = mma4(A[r16 * LK + kk + q4], sS[(16 * J + r16) * LS + kk + q4], acc);
                acc2 = mma4(A[r16 * LK + kk + 4 + q4], sS[(16 * J + r16) * LS + kk + 4 + q4], acc2);
            }
            acc += acc2;
            if (J == I && anyI) {
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) acc[ii] += sEx[which][4 * q4 + ii][r16];
            }
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int i = 16 * I + 4 * q4 + ii, j = 16 * J + r16;
                if (which == 0) {
                    const float val = j < i ? acc[ii] : 0.f;
                    sAp[i * LC + j] = val;
                    a.r.Ap[R * a.r.rs + i * C + j] = val;
                } else if (!SPLIT) {
                    sAqk[i * LQ + j] = j <= i ? acc[ii] : 0.f;
                }
            }
            if constexpr (SPLIT) {
                if (which == 1) {
                    // Aqk^T in bf16 parts: row j, the four columns i = 16 I + 4 q4 + ii
                    float x[4];
#pragma unroll
                    for (int ii = 0; ii < 4; ++ii) x[ii] = 16 * J + r16 <= 16 * I + 4 * q4 + ii ? acc[ii] : 0.f;
                    uint32_t h0, m0, l0, h1, m1, l1;
                    split3x2(x[0], x[1], h0, m0, l0);
                    split3x2(x[2], x[3], h1, m1, l1);
                    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
                    uint32_t* pq = reinterpret_cast<uint32_t*>(smem + S::oAqkP);
                    const int o = (16 * J + r16) * PW + 8 * I + 2 * q4;
                    *reinterpret_cast<u32x2_t*>(pq + o) = (u32x2_t){h0, h1};
                    *reinterpret_cast<u32x2_t*>(pq + C * PW + o) = (u32x2_t){m0, m1};
                    *reinterpret_cast<u32x2_t*>(pq + 2 * C * PW + o) = (u32x2_t){l0, l1};
                }
            }
        }
        lds_barrier();
    }

    // T = (I + A)^-1, A = Diag(beta) Ap: diagonal 16 x 16 blocks by column
    // substitution, then T_IJ = -T_II sum_{J <= K < I} A_IK T_KJ by block
    // distance on the matrix cores
    if (tid < 16 * NB) {
        // column `col` of the block, kept in registers; rows above the
        // diagonal come out zero by themselves
        const int base = 16 * (tid / 16), col = tid % 16;
        float t[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) {
            float s = 0.f;
#pragma unroll
            for (int j = 0; j < m; ++j) s += sAp[(base + m) * LC + base + j] * t[j];
            t[m] = (m == col ? 1.f : 0.f) - sBeta[base + m] * s;
        }
#pragma unroll
        for (int m = 0; m < 16; ++m) sT[(base + m) * LC + base + col] = t[m];
    }
    lds_barrier();
    for (int d = 1; d < NB; ++d) {
        if (w < NB - d) {
            const int J = w, I = w + d;
            const int i = 16 * I + r16;
            f32x4 M = zero4();
            for (int K = J; K < I; ++K) {
#pragma unroll
                for (int kk = 0; kk < 16; kk += 4)
                    M = mma4(sBeta[i] * sAp[i * LC + 16 * K + kk + q4],
                             sT[(16 * K + kk + q4) * LC + 16 * J + r16], M);
            }
            // M is the right operand as it stands: lane (r16, q4) holds M[4 q4 + s][r16]
            f32x4 acc = zero4();
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2)
                acc = mma4(sT[(16 * I + r16) * LC + 16 * I + 4 * q4 + s2], M[s2], acc);
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) sT[(16 * I + 4 * q4 + ii) * LC + 16 * J + r16] = -acc[ii];
        }
        lds_barrier();
    }
    for (int e = tid; e < C * C; e += NT) {
        const int i = e / C, j = e % C;
        a.r.Tm[R * a.r.rs + e] = (j >> 4) <= (i >> 4) ? sT[i * LC + j] : 0.f;
    }

    if constexpr (SPLIT) {
        // TB = T Diag(beta) in bf16 parts, rows of C values (blocks above the
        // diagonal zero); then (K e^G)^T in parts and V^T (exact)
        uint32_t* pTB = reinterpret_cast<uint32_t*>(smem + S::xTB);
        uint32_t* pKG = reinterpret_cast<uint32_t*>(smem + S::xKG);
        uint32_t* pVT = reinterpret_cast<uint32_t*>(smem + S::xVT);
        for (int g = tid; g < C * C / 8; g += NT) {
            const int i = g / (C / 8), j0 = 8 * (g % (C / 8));
            float x[8];
#pragma unroll
            for (int z = 0; z < 8; ++z)
                x[z] = (j0 >> 4) <= (i >> 4) ? sT[i * LC + j0 + z] * sBeta[j0 + z] : 0.f;
            put3x8(pTB, C * PW, i * PW + j0 / 2, x);
        }
        lds_barrier();
        {
            float x[RPT];
#pragma unroll
            for (int m = 0; m < RPT; ++m) x[m] = kr[m] * ex(Gr[m]);
#pragma unroll
            for (int g = 0; g < RPT; g += 8) put3x8(pKG, DK * PW, c * PW + (r0 + g) / 2, x + g);
            float y[RPV];
#pragma unroll
            for (int m = 0; m < RPV; ++m) y[m] = keep(vv[m], r0v + m, L);
#pragma unroll
            for (int g = 0; g < RPV; g += 8) put1x8(pVT, cv * PW + (r0v + g) / 2, y + g);
        }
        lds_barrier();
        // W = TB (K e^G) for the matrix-core state passes, in both
        // orientations: W [C][DK] (job (I, ks): tokens 16 I.., channels
        // 32 ks..) and W^T [DK][C] (job (Rc, kc): channels 16 Rc.., tokens
        // 32 kc..).  Each job forms the two 16 x 16 tiles of one fragment with
        // the operand whose rows are the fragment's k first, so that lane
        // (r16, q4) ends with its fragment values.  U = TB V, [DV][C].
        constexpr int KS = DK / 32, KC = C / 32;
        constexpr int NJ1 = NB * KS, NJ2 = (DK / 16) * KC, NJU = NB * (DV / 16);
        for (int job = w; job < NJ1 + NJ2 + NJU; job += NW) {
            if (job < NJ1) {
                const int I = job / KS, ks = job % KS;
                f32x4 acc[2] = {zero4(), zero4()};
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
                    for (int k0 = 0; k0 < 16 * (I + 1); k0 += 32)
                        acc[hh] = mm6(pfrag3(pKG + k0 / 2, DK * PW, PW, 32 * ks + 16 * hh + r16, q4),
                                      pfrag3(pTB + k0 / 2, C * PW, PW, 16 * I + r16, q4), acc[hh]);
                store_mc(reinterpret_cast<uint16_t*>(a.r.W + R * a.r.rs), C * DK,
                         ((I * KS + ks) * 64 + lane) * 8, acc[0], acc[1]);
            } else if (job < NJ1 + NJ2) {
                const int Rc = (job - NJ1) / KC, kc = (job - NJ1) % KC;
                f32x4 acc[2] = {zero4(), zero4()};
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int I = 2 * kc + hh;
                    for (int k0 = 0; k0 < 16 * (I + 1); k0 += 32)
                        acc[hh] = mm6(pfrag3(pTB + k0 / 2, C * PW, PW, 16 * I + r16, q4),
                                      pfrag3(pKG + k0 / 2, DK * PW, PW, 16 * Rc + r16, q4), acc[hh]);
                }
                store_mc(reinterpret_cast<uint16_t*>(a.r.WT + R * a.r.rs), C * DK,
                         ((Rc * KC + kc) * 64 + lane) * 8, acc[0], acc[1]);
            } else {
                const int ju = job - NJ1 - NJ2, I = ju / (DV / 16), Vt = ju % (DV / 16);
                f32x4 acc = zero4();
                for (int k0 = 0; k0 < 16 * (I + 1); k0 += 32)
                    acc = mm3b(pfrag3(pTB + k0 / 2, C * PW, PW, 16 * I + r16, q4),
                               pfrag(pVT + k0 / 2, PW, 16 * Vt + r16, q4), acc);
                *reinterpret_cast<f32x4*>(a.r.U + R * a.r.rs + (size_t)(16 * Vt + r16) * C + 16 * I + 4 * q4) = acc;
            }
        }
    } else {
        // W = T Diag(beta) (K e^G), stored as [C][DK] and transposed [DK][C]
    #pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int j = r0 + m;
            sS[j * LS + c] = sBeta[j] * kr[m] * ex(Gr[m]);
        }
        lds_barrier();
        for (int job = w; job < NB * (DK / 16); job += NW) {
            const int I = job / (DK / 16), Rc = job % (DK / 16);
            f32x4 acc = zero4();
            for (int kk = 0; kk < 16 * (I + 1); kk += 4)
                acc = mma4(sT[(16 * I + r16) * LC + kk + q4], sS[(kk + q4) * LS + 16 * Rc + r16], acc);
    #pragma unroll
            for (int ii = 0; ii < 4; ++ii)
                a.r.W[R * a.r.rs + (16 * I + 4 * q4 + ii) * DK + 16 * Rc + r16] = acc[ii];
            *reinterpret_cast<f32x4*>(a.r.WT + R * a.r.rs + (16 * Rc + r16) * C + 16 * I + 4 * q4) = acc;
        }
        lds_barrier();

        // U = T Diag(beta) V
    #pragma unroll
        for (int m = 0; m < RPV; ++m) {
            const int j = r0v + m;
            sS[j * LS + cv] = sBeta[j] * keep(vv[m], j, L);
        }
        lds_barrier();
        for (int job = w; job < NB * (DV / 16); job += NW) {
            const int I = job / (DV / 16), Rc = job % (DV / 16);
            f32x4 acc = zero4();
            for (int kk = 0; kk < 16 * (I + 1); kk += 4)
                acc = mma4(sT[(16 * I + r16) * LC + kk + q4], sS[(kk + q4) * LS + 16 * Rc + r16], acc);
            *reinterpret_cast<f32x4*>(a.r.U + R * a.r.rs + (size_t)(16 * Rc + r16) * C + 16 * I + 4 * q4) = acc;
        }

    }

    // Kr = K e^{G_last - G}, stored as [C][DK] and transposed [DK][C]
    if constexpr (SPLIT) {
        // in the matrix-core fragment order of the state passes: staged as
        // float32 [C][DK] over the operand planes of W and U (dead once every
        // wave is past the loop above), then read back a fragment lane at a time
        constexpr int LR = DK + 4, KS = DK / 32, KC = C / 32;
        static_assert(C * LR <= S::oAqkP, "staging clear of Aqk^T");
        float* const sKr = smem;
        lds_barrier();
#pragma unroll
        for (int m = 0; m < RPT; ++m) sKr[(r0 + m) * LR + c] = kr[m] * ex(sGref[NB][c] - Gr[m]);
        lds_barrier();
        uint16_t* const kb = reinterpret_cast<uint16_t*>(a.r.Kr + R * a.r.rs);
        uint16_t* const kt = reinterpret_cast<uint16_t*>(a.r.KrT + R * a.r.rs);
        constexpr int N1 = NB * KS * 64, N2 = (DK / 16) * KC * 64;
        for (int e = tid; e < N1 + N2; e += NT) {
            const int ln = e & 63, rr = ln & 15, gg = ln >> 4;
            f32x4 x0, x1;
            if (e < N1) {
                // Kr: fragment (token tile, channel step)
                const int f = e >> 6, rt = f / KS, ks = f % KS;
                const float* p = sKr + (16 * rt + rr) * LR + 32 * ks + 4 * gg;
                x0 = *reinterpret_cast<const f32x4*>(p);
                x1 = *reinterpret_cast<const f32x4*>(p + 16);
                store_mc(kb, C * DK, 8 * e, x0, x1);
            } else {
                // Kr^T: fragment (channel tile, token step)
                const int e2 = e - N1, f = e2 >> 6, rt = f / KC, kc = f % KC;
                const float* p = sKr + (32 * kc + 4 * gg) * LR + 16 * rt + rr;
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    x0[u] = p[u * LR];
                    x1[u] = p[(16 + u) * LR];
                }
                store_mc(kt, C * DK, 8 * e2, x0, x1);
            }
        }
    } else {
        float kx[RPT];
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            kx[m] = kr[m] * ex(sGref[NB][c] - Gr[m]);
            a.r.Kr[R * a.r.rs + (r0 + m) * DK + c] = kx[m];
        }
        float* kt = a.r.KrT + R * a.r.rs + (size_t)c * C + r0;
        if constexpr (RPT % 4 == 0) {
#pragma unroll
            for (int m = 0; m < RPT; m += 4)
                *reinterpret_cast<f32x4*>(kt + m) = (f32x4){kx[m], kx[m + 1], kx[m + 2], kx[m + 3]};
        } else {
#pragma unroll
            for (int m = 0; m < RPT; ++m) kt[m] = kx[m];
        }
    }
    lds_barrier();

    if constexpr (SPLIT) {
        // phase 2: Ut = Aqk^T dO [C][DV] and P = (scale Q e^G)^T dO [DK][DV] over
        // (scale Q e^G)^T in parts and dO^T (exact)
        uint32_t* pQG = reinterpret_cast<uint32_t*>(smem + S::yQG);
        uint32_t* pdO = reinterpret_cast<uint32_t*>(smem + S::ydO);
        const uint32_t* pAq = reinterpret_cast<const uint32_t*>(smem + S::oAqkP);
        {
            float x[RPT];
#pragma unroll
            for (int m = 0; m < RPT; ++m) x[m] = a.scale * qr[m] * ex(Gr[m]);
#pragma unroll
            for (int g = 0; g < RPT; g += 8) put3x8(pQG, DK * PW, c * PW + (r0 + g) / 2, x + g);
            float y[RPV];
#pragma unroll
            for (int m = 0; m < RPV; ++m) y[m] = keep(dv_[m], r0v + m, L);
#pragma unroll
            for (int g = 0; g < RPV; g += 8) put1x8(pdO, cv * PW + (r0v + g) / 2, y + g);
        }
        lds_barrier();
        constexpr int NJU = NB * (DV / 16), NJP = (DK / 16) * (DV / 16);
        for (int job = w; job < NJU + NJP; job += NW) {
            f32x4 acc = zero4();
            if (job < NJU) {
                // rows i >= 16 J; a step from 16 (J - 1) reads the zeroed block
                const int J = job / (DV / 16), Vt = job % (DV / 16);
                for (int k0 = 32 * (J / 2); k0 < C; k0 += 32)
                    acc = mm3b(pfrag3(pAq + k0 / 2, C * PW, PW, 16 * J + r16, q4),
                               pfrag(pdO + k0 / 2, PW, 16 * Vt + r16, q4), acc);
                *reinterpret_cast<f32x4*>(a.r.Ut + R * a.r.rs + (size_t)(16 * Vt + r16) * C + 16 * J + 4 * q4) = acc;
            } else {
                const int jp = job - NJU, Rc = jp / (DV / 16), Vt = jp % (DV / 16);
#pragma unroll
                for (int k0 = 0; k0 < C; k0 += 32)
                    acc = mm3b(pfrag3(pQG + k0 / 2, DK * PW, PW, 16 * Rc + r16, q4),
                               pfrag(pdO + k0 / 2, PW, 16 * Vt + r16, q4), acc);
                *reinterpret_cast<f32x4*>(a.r.P + R * a.r.rs + (size_t)(16 * Vt + r16) * DK + 16 * Rc + 4 * q4) = acc;
            }
        }
    } else {
        // phase 2: Ut = Aqk^T dO [C][DV] and P = (scale Q e^G)^T dO [DK][DV]
    #pragma unroll
        for (int m = 0; m < RPV; ++m) sdO[(r0v + m) * LO + cv] = keep(dv_[m], r0v + m, L);
    #pragma unroll
        for (int m = 0; m < RPT; ++m) sQg[(r0 + m) * LG + c] = a.scale * qr[m] * ex(Gr[m]);
        lds_barrier();
        constexpr int NJU = NB * (DV / 16), NJP = (DK / 16) * (DV / 16);
        for (int job = w; job < NJU + NJP; job += NW) {
            f32x4 acc = zero4();
            if (job < NJU) {
                const int J = job / (DV / 16), Vt = job % (DV / 16);
                for (int kk = 16 * J; kk < C; kk += 4)
                    acc = mma4(sAqk[(kk + q4) * LQ + 16 * J + r16], sdO[(kk + q4) * LO + 16 * Vt + r16], acc);
                *reinterpret_cast<f32x4*>(a.r.Ut + R * a.r.rs + (size_t)(16 * Vt + r16) * C + 16 * J + 4 * q4) = acc;
            } else {
                const int jp = job - NJU, Rc = jp / (DV / 16), Vt = jp % (DV / 16);
    #pragma unroll 8
                for (int kk = 0; kk < C; kk += 4)
                    acc = mma4(sQg[(kk + q4) * LG + 16 * Rc + r16], sdO[(kk + q4) * LO + 16 * Vt + r16], acc);
                *reinterpret_cast<f32x4*>(a.r.P + R * a.r.rs + (size_t)(16 * Vt + r16) * DK + 16 * Rc + 4 * q4) = acc;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// 2. sequential state passes (forward carry and reverse gradient carry)
// ---------------------------------------------------------------------------
// Workgroup = (head, 16-column value tile); wave w owns key channels
// [w CPW, (w + 1) CPW) and keeps their 16-column state strip in registers
// for the whole pass: lane (r16, q4) holds rows w CPW + q4 SQ + s, s < SQ,
// of column r16.  A product over key channels (E = U - W H, or
// dE = Ut + Kr dH) is a partial sum per wave, exchanged through LDS; the
// update of the wave's own rows (H' = Diag(gamma) H + Kr^T E, or
// dH = Diag(gamma) dH' + P - W^T dE) contracts over the chunk's rows with the
// output rows ordered so that each accumulator element lands on the lane
// and slot that holds that row of the strip.
template <int C, int DK>
struct StateShape {
    static constexpr int NB = C / 16;
    static constexpr int NWS = DK >= 64 ? 4 : DK / 16;   // waves
    static constexpr int CPW = DK / NWS;                  // key channels per wave: 16 or 32
    static constexpr int SQ = CPW / 4;                    // strip slots per lane
    static constexpr int TPW = CPW / 16;                  // 16-row tiles per wave
    static constexpr int CQ = C / 4;                      // chunk rows per lane group
    static constexpr int LP = C + 4;
};

template <int C, int DK, int DV, typename IO>
__global__ void __launch_bounds__(256) bwd_states(Args a)
{
    using S = StateShape<C, DK>;
    constexpr int NB = S::NB, NWS = S::NWS, CPW = S::CPW, SQ = S::SQ, TPW = S::TPW, CQ = S::CQ,
                  LP = S::LP;
    __shared__ __align__(16) float sPart[NWS][16][LP];   // per-wave partial sums, [column][row]
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r16 = lane & 15, q4 = lane >> 4;
    const int units = (a.stab ? a.N : a.B) * a.H;   // (sequence, head) pairs
    // Workgroups are handed to the eight XCDs round-robin by id; the DV / 16
    // value tiles of one (role, head) take ids 8 apart, so they share an XCD
    // and its L2, which then serves the records they all read.
    constexpr int NVT = DV / 16;
    const int L8 = blockIdx.x, xcd = L8 % 8, slot = L8 / 8;
    const int ur = (slot / NVT) * 8 + xcd, vt = slot % NVT;
    if (ur >= 2 * units) return;
    const bool reverse = ur >= units;
    const int u = reverse ? ur - units : ur;
    const int v0 = vt * 16;
    const size_t DD = (size_t)DK * DV;
    const int cw0 = w * CPW;
    // chunks of this (sequence, head): records R = rbase + rstep * chunk
    int NC;
    size_t rbase, rstep;
    if (a.stab) {
        const int4 sq = a.stab[u / a.H];
        NC = (sq.y + C - 1) / C;
        rbase = (size_t)(u % a.H) * a.Gmax + sq.z;
        rstep = 1;
    } else {
        NC = a.NC;
        rbase = (size_t)u * a.NC;
        rstep = 1;
    }
    // Strip slot s = 4 j + z of lane (r16, q4) holds key channel
    // cw0 + 16 j + 4 q4 + z, and output tile t of the strip update covers
    // channels cw0 + 16 t .. + 15 in order: the accumulator element ii of
    // tile t is then slot 4 t + ii, and every per-lane vector access below
    // reads 16 bytes of a 64-byte run shared with the three other lane groups.
    const int cbase = cw0 + 4 * q4;
    auto chan = [&](int s) { return cbase + 16 * (s >> 2) + (s & 3); };

    float st[SQ];
    {
        const float* init = reverse ? a.dhT : a.h0;
#pragma unroll
        for (int s = 0; s < SQ; ++s)
            st[s] = init ? init[(size_t)u * DD + (size_t)chan(s) * DV + v0 + r16] : 0.f;
    }

    // record bases of this role
    const float* const A1b = reverse ? a.r.Kr : a.r.W;     // rows 16 I + r16, this wave's channels
    const float* const A2b = reverse ? a.r.WT : a.r.KrT;   // rows of this wave's output tiles
    const float* const ADb = reverse ? a.r.Ut : a.r.U;     // added to the partial sums (wave 0)
    float* const recb = reverse ? a.r.dH : a.r.Hs;
    float* const erb = reverse ? a.r.dE : a.r.E;

    // operands used at the start of a step: requested one step ahead, in two
    // sets that alternate (registers are scarce: the strip update's operands
    // are requested later, see load_A2 and step)
    struct Pre {
        float A1[NB][SQ];
        float add[(NB + NWS - 1) / NWS][4];   // U or Ut of blocks w, w + NWS, ...
    };
    auto load_pre = [&](Pre& o, int ch) {
        const size_t R = rbase + rstep * ch;
#pragma unroll
        for (int I = 0; I < NB; ++I) {
            const float* p = A1b + R * a.r.rs + (16 * I + r16) * DK + cbase;
#pragma unroll
            for (int s = 0; s < SQ; s += 4) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(p + 4 * s);
                o.A1[I][s] = x[0]; o.A1[I][s + 1] = x[1]; o.A1[I][s + 2] = x[2]; o.A1[I][s + 3] = x[3];
            }
        }
        // the term added to the partial sums of block I is added by wave
        // I % NWS, so each wave holds a quarter of it (with four waves)
#pragma unroll
        for (int j = 0; j < (NB + NWS - 1) / NWS; ++j) {
            const int I = min(w + j * NWS, NB - 1);
            const f32x4 x = *reinterpret_cast<const f32x4*>(ADb + R * a.r.rs + (size_t)(v0 + r16) * C + 16 * I + 4 * q4);
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) o.add[j][ii] = x[ii];
        }
    };

    // one chunk step with its early operands in `cur`
    auto chunk_of = [&](int n) { return reverse ? max(NC - 1 - n, 0) : min(n, NC - 1); };

    // the strip update's matrix operand (Kr^T or W^T rows of this wave's
    // output tiles): requested at the end of the previous step, into the
    // registers that step's update has just released
    float A2[TPW][CQ];
    auto load_A2 = [&](int ch) {
        const size_t R = rbase + rstep * ch;
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const float* p = A2b + R * a.r.rs + (size_t)(cw0 + 16 * t + r16) * C + 4 * q4;
#pragma unroll
            for (int s = 0; s < CQ; s += 4) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(p + 4 * s);
                A2[t][s] = x[0]; A2[t][s + 1] = x[1]; A2[t][s + 2] = x[2]; A2[t][s + 3] = x[3];
            }
        }
    };

    // one chunk step with its early operands in `cur`; it requests the next
    // step's into `nxt` right after its own small update operands, and the
    // next update operand at its end (loads complete in order, so no wait for
    // an operand covers a load issued after it)
    auto step = [&](const Pre& cur, Pre& nxt, int n) {
        const int ch = reverse ? NC - 1 - n : n;
        const size_t R = rbase + rstep * ch;
        // gates and P of the strip update, first used after the exchange
        float gam[SQ], Pv[SQ];
        {
            const float* Gl = a.r.G + R * a.r.rs + (C - 1) * DK + cbase;
            const float* P = a.r.P + R * a.r.rs + (size_t)(v0 + r16) * DK + cbase;
#pragma unroll
            for (int s = 0; s < SQ; s += 4) {
                const f32x4 x = *reinterpret_cast<const f32x4*>(Gl + 4 * s);
                gam[s] = x[0]; gam[s + 1] = x[1]; gam[s + 2] = x[2]; gam[s + 3] = x[3];
                if (reverse) {
                    const f32x4 y = *reinterpret_cast<const f32x4*>(P + 4 * s);
                    Pv[s] = y[0]; Pv[s + 1] = y[1]; Pv[s + 2] = y[2]; Pv[s + 3] = y[3];
                } else {
                    Pv[s] = Pv[s + 1] = Pv[s + 2] = Pv[s + 3] = 0.f;
                }
            }
        }

        load_pre(nxt, chunk_of(n + 1));

        // the state entering the chunk (forward) or the gradient leaving it (reverse)
        float* rec = recb + R * a.r.rs + (size_t)(v0 + r16) * DK + cbase;
#pragma unroll
        for (int s = 0; s < SQ; s += 4)
            *reinterpret_cast<f32x4*>(rec + 4 * s) = (f32x4){st[s], st[s + 1], st[s + 2], st[s + 3]};

        // partial sums over this wave's channels
#pragma unroll
        for (int I = 0; I < NB; ++I) {
            f32x4 acc = zero4();
#pragma unroll
            for (int s = 0; s < SQ; ++s) acc = mma4(cur.A1[I][s], st[s], acc);
            f32x4 part;
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                // forward: E = U - sum_w (W H)_w ; reverse: dE = Ut + sum_w (Kr dH)_w
                const float x = reverse ? acc[ii] : -acc[ii];
                part[ii] = I % NWS == w ? cur.add[I / NWS][ii] + x : x;
            }
            *reinterpret_cast<f32x4*>(&sPart[w][r16][16 * I + 4 * q4]) = part;
        }
        lds_barrier();
        float e[CQ];
        constexpr int HB = CQ / 4 > 1 ? CQ / 8 : 1;     // f32x4 groups read per batch
#pragma unroll
        for (int s0 = 0; s0 < CQ / 4; s0 += HB) {
            f32x4 pv[NWS][HB];
#pragma unroll
            for (int ww = 0; ww < NWS; ++ww) {
#pragma unroll
                for (int s = 0; s < HB; ++s)
                    pv[ww][s] = *reinterpret_cast<const f32x4*>(&sPart[ww][r16][16 * (s0 + s) + 4 * q4]);
            }
#pragma unroll
            for (int s = 0; s < HB; ++s) {
                f32x4 x = pv[0][s];
#pragma unroll
                for (int ww = 1; ww < NWS; ++ww) x += pv[ww][s];
                const int b4 = 4 * (s0 + s);
                e[b4] = x[0]; e[b4 + 1] = x[1]; e[b4 + 2] = x[2]; e[b4 + 3] = x[3];
            }
        }
        if (w == 0) {
            float* er = erb + R * a.r.rs + (size_t)(v0 + r16) * C + 4 * q4;
#pragma unroll
            for (int s = 0; s < CQ; s += 4)
                *reinterpret_cast<f32x4*>(er + 4 * s) = (f32x4){e[s], e[s + 1], e[s + 2], e[s + 3]};
        }
        // update of this wave's strip
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            f32x4 acc = zero4();
#pragma unroll
            for (int s = 0; s < CQ; ++s) acc = mma4(A2[t][s], e[s], acc);
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int s = 4 * t + ii;
                const float gm = ex(gam[s]);
                st[s] = reverse ? gm * st[s] + Pv[s] - acc[ii] : gm * st[s] + acc[ii];
            }
        }
        load_A2(chunk_of(n + 1));
        lds_barrier();
    };

    // two sets of early operands in turn, so a prefetch is consumed a whole
    // step after it was issued and never copied
    Pre bufA, bufB;
    if (NC > 0) {
        load_pre(bufA, chunk_of(0));
        load_A2(chunk_of(0));
    }
    for (int n = 0; n < NC; n += 2) {
        step(bufA, bufB, n);
        if (n + 1 < NC) step(bufB, bufA, n + 1);
    }
    if (reverse && a.dh0) {
#pragma unroll
        for (int s = 0; s < SQ; ++s) a.dh0[(size_t)u * DD + (size_t)chan(s) * DV + v0 + r16] = st[s];
    }
}

// The same two carries on the bf16 matrix cores, for bf16 inputs (where
// bwd_prep stores W, W^T, Kr and Kr^T as bf16 pairs in the fragment order of
// store_mc).  Every product is hi*hi + hi*lo + lo*hi of the pairs (mma3),
// good to about 2^-16 of its operands, against float32 products in
// bwd_states; the carried state stays in float32 accumulators.
//
// Workgroup = (role, sequence-head, 16 value columns), four waves.  Wave w
// computes token tile w of E = U - W H (forward) or dE = Ut + Kr dH'
// (reverse) over all key channels, with the state's 16 columns read from LDS
// as the right operand; after the barrier it updates state tiles w, w + 4, ..
// with Kr^T E (or P - W^T dE) over the chunk's tokens, E read from LDS.  Two
// barriers per chunk; the next chunk's operands are requested at the start of
// each step.
template <int C, int DK, int DV, int NT2>
__global__ void __launch_bounds__(256) bwd_states_mc(Args a)
{
    constexpr int NB = C / 16, KS = DK / 32, KC = C / 32, MH = DK / 16, MHW = MH / 4;
    constexpr int NCOL = 16 * NT2;              // value columns of one workgroup (NT2 16-column tiles)
    constexpr int SK = DK + 8, SC = C + 8;      // LDS row strides (bf16 elements)
    constexpr int PL = C * DK;                  // elements per bf16 plane of a record operand
    static_assert(DK % 64 == 0 && DK <= 128 && C % 32 == 0, "whole fragments for every wave, at most two state tiles");
    static_assert(DV % NCOL == 0, "whole tiles per workgroup");
    __shared__ __align__(16) bf16_t HTs[2 * NCOL * SK];   // state^T [column][channel], hi and lo
    __shared__ __align__(16) bf16_t ETs[2 * NCOL * SC];   // E^T [column][token], hi and lo
    const PArr<bf16_t> HT{HTs, HTs + NCOL * SK};
    const PArr<bf16_t> ET{ETs, ETs + NCOL * SC};

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int units = (a.stab ? a.N : a.B) * a.H;
    // XCD-aware: the DV / NCOL workgroups of one (role, head) take ids 8
    // apart, so they share an XCD and its L2, which serves their common records
    constexpr int NVT = DV / NCOL;
    const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
    const int ur = (slot / NVT) * 8 + xcd, vt = slot % NVT;
    if (ur >= 2 * units) return;
    const bool reverse = ur >= units;
    const int u = reverse ? ur - units : ur;
    const int v0 = vt * NCOL;
    const size_t DD = (size_t)DK * DV;
    int NC;
    size_t rbase;
    if (a.stab) {
        const int4 sq = a.stab[u / a.H];
        NC = (sq.y + C - 1) / C;
        rbase = (size_t)(u % a.H) * a.Gmax + sq.z;
    } else {
        NC = a.NC;
        rbase = (size_t)u * a.NC;
    }
    const bool has_t = w < NB;                  // this wave owns a token tile
    const int we = has_t ? w : NB - 1;

    // the state strip: accumulator [s][n] holds rows 16 (w + 4 s) + 4 g + 0..3
    // of column v0 + 16 n + r
    f32x4 hacc[MHW][NT2];
    {
        const float* init = reverse ? a.dhT : a.h0;
#pragma unroll
        for (int s = 0; s < MHW; ++s) {
            const int mt = w + 4 * s;
#pragma unroll
            for (int n = 0; n < NT2; ++n) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    hacc[s][n][e] = init ? init[(size_t)u * DD + (size_t)(16 * mt + 4 * g + e) * DV + v0 + 16 * n + r]
                                         : 0.f;
                store4_p(HT, (16 * n + r) * SK + 32 * (mt >> 1) + mc_pos(16 * (mt & 1) + 4 * g), hacc[s][n]);
            }
        }
    }
    __syncthreads();

    const float* const A1b = reverse ? a.r.Kr : a.r.W;     // [C][DK] fragments, token tile we
    const float* const A2b = reverse ? a.r.WT : a.r.KrT;   // [DK][C] fragments, state tiles
    const float* const ADb = reverse ? a.r.Ut : a.r.U;
    float* const recb = reverse ? a.r.dH : a.r.Hs;
    float* const erb = reverse ? a.r.dE : a.r.E;

    // operands of one chunk step: the fragments and the gate row are shared
    // by the workgroup's tiles, U (or Ut) and P are per tile
    struct Ops {
        PFrag<bf16_t> a1[KS];
        PFrag<bf16_t> a2[MHW][KC];
        f32x4 add[NT2];
        f32x4 p[MHW][NT2];
        float gl;        // G_last of one channel of this lane's row (see oGl1)
    };
    // Record fields are addressed as a uniform record base plus per-lane
    // 32-bit byte offsets fixed for the whole pass, so that every load takes
    // its address from scalar registers and one loop-invariant vector offset
    // (tile n of a workgroup adds a constant).
    const char* const wsb = reinterpret_cast<const char*>(a.r.G);
    const uint32_t fA1 = (uint32_t)(reinterpret_cast<const char*>(A1b) - wsb);
    const uint32_t fA2 = (uint32_t)(reinterpret_cast<const char*>(A2b) - wsb);
    const uint32_t fAD = (uint32_t)(reinterpret_cast<const char*>(ADb) - wsb);
    const uint32_t fP = (uint32_t)(reinterpret_cast<const char*>(a.r.P) - wsb);
    const uint32_t oAdd = fAD + 4u * (uint32_t)((v0 + r) * C + 16 * we + 4 * g);
    const uint32_t oA1 = fA1 + 16u * (uint32_t)(we * KS * 64 + lane);
    const uint32_t oA2 = fA2 + 16u * (uint32_t)(w * KC * 64 + lane);
    // the last gate row: lane (r, g) loads channel 16 (w + 4 s) + 4 g + e for
    // r = 4 s + e (r mod 8), and lane 4 s + e of each 16-lane row then hands
    // it to the whole row (every lane of a row needs the same eight values)
    const uint32_t oGl1 =
        4u * (uint32_t)((C - 1) * DK + 16 * (w + 4 * ((r >> 2) & (MHW - 1))) + 4 * g + (r & 3));
    // P, added on the reverse role only: the forward role reads it through a
    // resource of zero length, which returns zeros without a memory access
    const uint32_t oP = fP + 4u * (uint32_t)((v0 + r) * DK + 16 * w + 4 * g);
    const int pbytes = reverse ? 0x7fffffff : 0;
    const uint32_t oRec = (uint32_t)(reinterpret_cast<const char*>(recb) - wsb) + 4u * (uint32_t)((v0 + r) * DK + 16 * w + 4 * g);
    const uint32_t oE = (uint32_t)(reinterpret_cast<const char*>(erb) - wsb) + 4u * (uint32_t)((v0 + r) * C + 16 * we + 4 * g);
    auto load_ops = [&](Ops& o, int ch) {
        const char* const base = wsb + (rbase + (size_t)ch) * a.r.rs * sizeof(float);
        const __amdgpu_buffer_rsrc_t rb = record_rsrc(base);
        const __amdgpu_buffer_rsrc_t rp = record_rsrc(base, pbytes);
#pragma unroll
        for (int n = 0; n < NT2; ++n) o.add[n] = bload<f32x4>(rb, oAdd, 64 * C * n);
        o.gl = bload1(rb, oGl1, 0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            o.a1[ks].h.v = bload<u16x8>(rb, oA1, 1024 * ks);
            o.a1[ks].l.v = bload<u16x8>(rb, oA1, 2 * PL + 1024 * ks);
        }
#pragma unroll
        for (int s = 0; s < MHW; ++s) {
            // state tile w + 4 s: 64 channels further on
#pragma unroll
            for (int n = 0; n < NT2; ++n) o.p[s][n] = bload<f32x4>(rp, oP, 256 * s + 64 * DK * n);
#pragma unroll
            for (int kc = 0; kc < KC; ++kc) {
                o.a2[s][kc].h.v = bload<u16x8>(rb, oA2, 1024 * (4 * s * KC + kc));
                o.a2[s][kc].l.v = bload<u16x8>(rb, oA2, 2 * PL + 1024 * (4 * s * KC + kc));
            }
        }
    };
    auto chunk_of = [&](int n) { return reverse ? max(NC - 1 - n, 0) : min(n, NC - 1); };
    // one tile: three operand sets in rotation, a chunk's operands requested
    // two steps before their use; two tiles: two sets, one step ahead (a
    // third does not fit the registers)
    constexpr int AHEAD = NT2 == 1 ? 2 : 1;

    auto step = [&](const Ops& P, Ops& Q, int n) {
        char* const rb = const_cast<char*>(wsb) + (rbase + (size_t)chunk_of(n)) * a.r.rs * sizeof(float);
        load_ops(Q, chunk_of(n + AHEAD));
        // the state entering the chunk (forward) or the gradient leaving it (reverse)
#pragma unroll
        for (int s = 0; s < MHW; ++s) {
#pragma unroll
            for (int t = 0; t < NT2; ++t)
                *reinterpret_cast<f32x4*>(rb + oRec + 256u * s + 64u * DK * t) = hacc[s][t];
        }
        if (has_t) {
            f32x4 ea[NT2], eb[NT2];
#pragma unroll
            for (int t = 0; t < NT2; ++t) {
                ea[t] = zero4();
                eb[t] = zero4();
            }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
                for (int t = 0; t < NT2; ++t) {
                    const PFrag<bf16_t> hf = HT.frag((16 * t + r) * SK + 32 * ks + 8 * g);
                    if (ks & 1) eb[t] = mma3(P.a1[ks], hf, eb[t]);
                    else ea[t] = mma3(P.a1[ks], hf, ea[t]);
                }
            }
#pragma unroll
            for (int t = 0; t < NT2; ++t) {
                const f32x4 e = reverse ? P.add[t] + (ea[t] + eb[t]) : P.add[t] - (ea[t] + eb[t]);
                store4_p(ET, (16 * t + r) * SC + 32 * (we >> 1) + mc_pos(16 * (we & 1) + 4 * g), e);
                *reinterpret_cast<f32x4*>(rb + oE + 64u * C * t) = e;
            }
        }
        lds_barrier();
        float gm[MHW][4];
        {
            const float egl = ex(P.gl);
            gm[0][0] = row_bcast<0>(egl); gm[0][1] = row_bcast<1>(egl);
            gm[0][2] = row_bcast<2>(egl); gm[0][3] = row_bcast<3>(egl);
            if constexpr (MHW > 1) {
                gm[MHW - 1][0] = row_bcast<4>(egl); gm[MHW - 1][1] = row_bcast<5>(egl);
                gm[MHW - 1][2] = row_bcast<6>(egl); gm[MHW - 1][3] = row_bcast<7>(egl);
            }
        }
#pragma unroll
        for (int s = 0; s < MHW; ++s) {
            const int mt = w + 4 * s;
#pragma unroll
            for (int t = 0; t < NT2; ++t) {
                f32x4 xa = zero4(), xb = zero4();
#pragma unroll
                for (int kc = 0; kc < KC; ++kc) {
                    const PFrag<bf16_t> ef = ET.frag((16 * t + r) * SC + 32 * kc + 8 * g);
                    if (kc & 1) xb = mma3(P.a2[s][kc], ef, xb);
                    else xa = mma3(P.a2[s][kc], ef, xa);
                }
                const f32x4 x = xa + xb;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    hacc[s][t][e] = gm[s][e] * hacc[s][t][e] + P.p[s][t][e] + (reverse ? -x[e] : x[e]);
                store4_p(HT, (16 * t + r) * SK + 32 * (mt >> 1) + mc_pos(16 * (mt & 1) + 4 * g), hacc[s][t]);
            }
        }
        lds_barrier();
    };

    if constexpr (NT2 == 1) {
        Ops bufA, bufB, bufC;
        if (NC > 0) {
            load_ops(bufA, chunk_of(0));
            load_ops(bufB, chunk_of(1));
        }
        for (int n = 0; n < NC; n += 3) {
            step(bufA, bufC, n);
            if (n + 1 < NC) step(bufB, bufA, n + 1);
            if (n + 2 < NC) step(bufC, bufB, n + 2);
        }
    } else {
        Ops bufA, bufB;
        if (NC > 0) load_ops(bufA, chunk_of(0));
        for (int n = 0; n < NC; n += 2) {
            step(bufA, bufB, n);
            if (n + 1 < NC) step(bufB, bufA, n + 1);
        }
    }
    if (reverse && a.dh0) {
#pragma unroll
        for (int s = 0; s < MHW; ++s) {
            const int mt = w + 4 * s;
#pragma unroll
            for (int t = 0; t < NT2; ++t) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    a.dh0[(size_t)u * DD + (size_t)(16 * mt + 4 * g + e) * DV + v0 + 16 * t + r] = hacc[s][t][e];
            }
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
    // row strides (floats): 16 mod 32 where lanes run along a row, 2 mod 32
    // where they run down a column
    static constexpr int LT = C + 16, LV = VS + 2, LA = C + 2;
    static constexpr int LHT = (DK + 31) / 32 * 32 + 16, LET = (C + 31) / 32 * 32 + 16, LDE = C + 2;
    // value-slice phase; the state, its gradient and E are kept transposed
    // ([value column][row]) as the records hold them
    static constexpr int oT = 0, oH = oT + C * LT, odH = oH + VS * LHT, oE = odH + VS * LHT,
                         odO = oE + VS * LET, odU = odO + C * LV, oV = odU + C * LV,
                         odE = oV + C * LV, S_END = odE + VS * LDE;
    // value-slice phase with split bf16 operands (slices of 32 columns):
    // float T, V and dE (transposed), then bf16 planes [row][SB] of the
    // hi, mid and lo parts of the state, its gradient, E, dO and dUt
    // (offsets in floats)
    static constexpr bool SPLIT = VS == 32;
    static constexpr int SB = VS + 8;
    static constexpr int hT = 0, hV = hT + C * LT, hdE = hV + C * LV, hP = hdE + VS * LDE;
    static constexpr int pH = DK * SB / 2, pC = C * SB / 2;   // floats per plane
    static constexpr int hH = hP, hdH = hH + 3 * pH, hE = hdH + 3 * pH, hO = hE + 3 * pC,
                         hU = hO + 3 * pC, H_END = hU + 3 * pC;
    static constexpr int SL_END = SPLIT ? H_END : S_END;
    // output phase
    static constexpr int oAq = 0, oAb = oAq + C * LA, oSrc = oAb + C * LA,
                         oRow = oSrc + NW * 2 * C * 16, oRowG = oRow + NW * C,
                         E_END = oRowG + NW * C;
    static constexpr int SIZE = SL_END > E_END ? SL_END : E_END;
};

template <int C, int DK, int DV, typename IO>
__global__ void __launch_bounds__(4 * DK) bwd_grad(Args a)
{
    using S = GradLds<C, DK, DV>;
    constexpr int NB = S::NB, NW = S::NW, NT = 64 * NW;
    constexpr int VS = S::VS, NS = DV / VS;
    constexpr int LT = S::LT, LV = S::LV, LA = S::LA, LHT = S::LHT, LET = S::LET, LDE = S::LDE;
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
    const ChunkLoc loc = locate_chunk<C>(a, rec);
    if (loc.L <= 0) return;                  // empty slot of a packed batch
    const int b = loc.b, h = loc.h, hq = h / (a.H / a.Hq);
    const int t0 = loc.t0;
    const int L = loc.L;
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

    {
        constexpr int NTT = (C * C / 4 + NT - 1) / NT;
        f32x4 tv[NTT];
#pragma unroll
        for (int j = 0; j < NTT; ++j)
            tv[j] = *reinterpret_cast<const f32x4*>(a.r.Tm + R * a.r.rs + 4 * min(tid + j * NT, C * C / 4 - 1));
#pragma unroll
        for (int j = 0; j < NTT; ++j) {
            const int e = 4 * (tid + j * NT);
            if (e < C * C) *reinterpret_cast<f32x4*>(sT + (e / C) * LT + e % C) = tv[j];
        }
    }
    for (int i = tid; i < C; i += NT) sBeta[i] = i < L ? a.beta[tok_v(a, b, t0 + i, h)] : 0.f;
    for (int e = tid; e < C * NB; e += NT) sPart[e / NB][e % NB] = 0.f;

    f32x4 X1[NB], X2[NB], X3[NB], Y[NYS];
#pragma unroll
    for (int I = 0; I < NB; ++I) { X1[I] = zero4(); X2[I] = zero4(); X3[I] = zero4(); }
#pragma unroll
    for (int s = 0; s < NYS; ++s) Y[s] = zero4();
    float zacc = 0.f, gacc = 0.f;

    if constexpr (S::SPLIT) {
        // Slices of 32 value columns: every product of the slice is a sum of
        // 32-deep steps of v_mfma_f32_16x16x32_bf16 over bf16 parts of the
        // float32 operands, x = x_h + x_m + x_l.  A product keeps the parts
        // down to 2^-24 of the operands (hh + hm + mh + hl + lh + mm, six
        // steps); dO of a bf16 batch is exact in bf16 and takes three steps
        // (h against h, m, l).  dUt H^T keeps hh + hm + mh: its error
        // (2^-16 of the products) only reaches dk and dG through Pg, where
        // it stays far below the float32 tolerance.  Operand convention of
        // that instruction (lane l, r = l % 16, g = l / 16): A[r][8g..8g+7],
        // B[8g..8g+7][r]; the accumulator is laid out as for the float32
        // instruction.  Planes hold bf16 rows of 32 columns (stride SB); the
        // state, its gradient and E are transposed on the way in, two value
        // columns per 32-bit write.
        constexpr int SB = S::SB, SW = SB / 2, PH = S::pH, PC = S::pC;
        constexpr bool OEX = std::is_same<IO, bf16_t>::value;
        uint32_t* pH = reinterpret_cast<uint32_t*>(smem + S::hH);     // + m * PH
        uint32_t* pdH = reinterpret_cast<uint32_t*>(smem + S::hdH);
        uint32_t* pE = reinterpret_cast<uint32_t*>(smem + S::hE);     // + m * PC
        uint32_t* pO = reinterpret_cast<uint32_t*>(smem + S::hO);
        uint32_t* pU = reinterpret_cast<uint32_t*>(smem + S::hU);
        float* sVh = smem + S::hV;
        float* sdEh = smem + S::hdE;
        // the three parts of a pair of values into three planes of PS floats
        auto put3 = [&](uint32_t* plane, int PS, int o, float x0, float x1) {
            uint32_t h, m, l;
            split3x2(x0, x1, h, m, l);
            plane[o] = h;
            plane[PS + o] = m;
            plane[2 * PS + o] = l;
        };
        auto frag = [&](const uint32_t* plane, int row) -> u16x8 { return pfrag(plane, SW, row, q4); };
        auto frag3 = [&](const uint32_t* plane, int PS, int row) -> F3 { return pfrag3(plane, PS, SW, row, q4); };
        // element maps (tid-based, 64-lane groups): a state or E element is
        // (column quad cq, value-column pair p), with four consecutive quads
        // per 64 bytes of a record row; a dO / v element is (row i, pair p)
        constexpr int NEP = 4 * C, NOP = 16 * C;
        constexpr int NEJ = (NEP + NT - 1) / NT, NOJ = (NOP + NT - 1) / NT;
        constexpr int NES = C * VS / 4, NE = (NES + NT - 1) / NT;
        static_assert(4 * DK == NT, "one state element pair per thread");
        const int hcq = 4 * (tid >> 6) + (tid & 3), hp = (tid >> 2) & 15;
        float gpart[4] = {0.f, 0.f, 0.f, 0.f};     // sum_n H dH of channels 4 hcq + z
        // sum_n dUt v of chunk rows, spread over all threads: element e is
        // (row e / 8, columns 4 (e % 8) .. + 3 of the slice)
        constexpr int NZ = (8 * C + NT - 1) / NT;
        float zpart[NZ];
#pragma unroll
        for (int j = 0; j < NZ; ++j) zpart[j] = 0.f;
        struct SliceS {
            f32x4 h0, h1, d0, d1, e0[NEJ], e1[NEJ], de[NE];
            float o0[NOJ], o1[NOJ], v0[NOJ], v1[NOJ];
        };
        auto load_slice = [&](SliceS& x, int s) {
            const int v0 = s * VS;
            {
                const size_t o = R * a.r.rs + (size_t)(v0 + 2 * hp) * DK + 4 * hcq;
                x.h0 = *reinterpret_cast<const f32x4*>(a.r.Hs + o);
                x.h1 = *reinterpret_cast<const f32x4*>(a.r.Hs + o + DK);
                x.d0 = *reinterpret_cast<const f32x4*>(a.r.dH + o);
                x.d1 = *reinterpret_cast<const f32x4*>(a.r.dH + o + DK);
            }
#pragma unroll
            for (int j = 0; j < NEJ; ++j) {
                const int e = min(tid + j * NT, NEP - 1);
                const int iq = 4 * (e >> 6) + (e & 3), p = (e >> 2) & 15;
                const size_t o = R * a.r.rs + (size_t)(v0 + 2 * p) * C + 4 * iq;
                x.e0[j] = *reinterpret_cast<const f32x4*>(a.r.E + o);
                x.e1[j] = *reinterpret_cast<const f32x4*>(a.r.E + o + C);
            }
#pragma unroll
            for (int j = 0; j < NE; ++j) {
                const int e = min(tid + j * NT, NES - 1);
                const int n = e / (C / 4), i = 4 * (e % (C / 4));
                x.de[j] = *reinterpret_cast<const f32x4*>(a.r.dE + R * a.r.rs + (size_t)(v0 + n) * C + i);
            }
#pragma unroll
            for (int j = 0; j < NOJ; ++j) {
                const int e = min(tid + j * NT, NOP - 1);
                const int i = clamp_row(e >> 4, L), p = e & 15;
                const size_t o = tok_v(a, b, t0 + i, h) * DV + v0 + 2 * p;
                if constexpr (OEX) {
                    // the bf16 pair stays packed until it is stored
                    x.o0[j] = __uint_as_float(*reinterpret_cast<const uint32_t*>(dO + o));
                    x.v0[j] = __uint_as_float(*reinterpret_cast<const uint32_t*>(v + o));
                } else {
                    const float2 fo = *reinterpret_cast<const float2*>(dO + o);
                    const float2 fv = *reinterpret_cast<const float2*>(v + o);
                    x.o0[j] = fo.x; x.o1[j] = fo.y;
                    x.v0[j] = fv.x; x.v1[j] = fv.y;
                }
            }
        };
        auto store_slice = [&](const SliceS& x) {
#pragma unroll
            for (int z = 0; z < 4; ++z) {
                const int o = (4 * hcq + z) * SW + hp;
                put3(pH, PH, o, x.h0[z], x.h1[z]);
                put3(pdH, PH, o, x.d0[z], x.d1[z]);
                gpart[z] += x.h0[z] * x.d0[z] + x.h1[z] * x.d1[z];
            }
#pragma unroll
            for (int j = 0; j < NEJ; ++j) {
                const int e = tid + j * NT;
                if (e < NEP) {
                    const int iq = 4 * (e >> 6) + (e & 3), p = (e >> 2) & 15;
#pragma unroll
                    for (int z = 0; z < 4; ++z) put3(pE, PC, (4 * iq + z) * SW + p, x.e0[j][z], x.e1[j][z]);
                }
            }
#pragma unroll
            for (int j = 0; j < NE; ++j) {
                const int e = tid + j * NT;
                if (e < NES) {
                    const int n = e / (C / 4), i = 4 * (e % (C / 4));
#pragma unroll
                    for (int z = 0; z < 4; ++z) sdEh[n * LDE + i + z] = x.de[j][z];
                }
            }
#pragma unroll
            for (int j = 0; j < NOJ; ++j) {
                const int e = tid + j * NT;
                if (e < NOP) {
                    const int i = e >> 4, p = e & 15;
                    if constexpr (OEX) {
                        const uint32_t uo = i < L ? __float_as_uint(x.o0[j]) : 0u;
                        const uint32_t uv = i < L ? __float_as_uint(x.v0[j]) : 0u;
                        pO[i * SW + p] = uo;
                        sVh[i * LV + 2 * p] = __uint_as_float(uv << 16);
                        sVh[i * LV + 2 * p + 1] = __uint_as_float(uv & 0xffff0000u);
                    } else {
                        put3(pO, PC, i * SW + p, keep(x.o0[j], i, L), keep(x.o1[j], i, L));
                        sVh[i * LV + 2 * p] = keep(x.v0[j], i, L);
                        sVh[i * LV + 2 * p + 1] = keep(x.v1[j], i, L);
                    }
                }
            }
        };

        SliceS nx;
        load_slice(nx, 0);
        uint16_t* pU16 = reinterpret_cast<uint16_t*>(pU);
        for (int s = 0; s < NS; ++s) {
            const int v0 = s * VS;
            lds_barrier();
            store_slice(nx);
            if (s + 1 < NS) load_slice(nx, s + 1);
            lds_barrier();
            // dUt = T^T dE (upper triangular: rows i take j >= 16 I), dv = beta dUt
            for (int job = w; job < NB * (VS / 16); job += NW) {
                const int I = job / (VS / 16), Vt = job % (VS / 16);
                f32x4 acc = zero4(), acc2 = zero4();   // two independent chains
                for (int kk = 16 * I; kk < C; kk += 8) {
                    acc = mma4(sT[(kk + q4) * LT + 16 * I + r16], sdEh[(16 * Vt + r16) * LDE + kk + q4], acc);
                    acc2 = mma4(sT[(kk + 4 + q4) * LT + 16 * I + r16],
                                sdEh[(16 * Vt + r16) * LDE + kk + 4 + q4], acc2);
                }
                acc += acc2;
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const int i = 16 * I + 4 * q4 + ii, n = 16 * Vt + r16;
                    uint16_t hi, mid, lo;
                    split3(acc[ii], hi, mid, lo);
                    pU16[i * SB + n] = hi;
                    pU16[2 * PC + i * SB + n] = mid;
                    pU16[4 * PC + i * SB + n] = lo;
                    if (i < L)
                        store_grad(a.dv, tok_v(a, b, t0 + i, h) * DV + v0 + n, sBeta[i] * acc[ii], a.gdt);
                }
            }
            lds_barrier();
#pragma unroll
            for (int j = 0; j < NZ; ++j) {
                const int e = tid + j * NT;
                if (e < 8 * C) {
                    const int i = e >> 3, p0 = 2 * (e & 7);
                    float z = 0.f;
#pragma unroll
                    for (int p = p0; p < p0 + 2; ++p) {
                        const uint32_t uh = pU[i * SW + p], um = pU[PC + i * SW + p],
                                       ul = pU[2 * PC + i * SW + p];
                        const float u0 = __uint_as_float(uh << 16) + __uint_as_float(um << 16) +
                                         __uint_as_float(ul << 16);
                        const float u1 = __uint_as_float(uh & 0xffff0000u) +
                                         __uint_as_float(um & 0xffff0000u) + __uint_as_float(ul & 0xffff0000u);
                        z += u0 * sVh[i * LV + 2 * p] + u1 * sVh[i * LV + 2 * p + 1];
                    }
                    zpart[j] += z;
                }
            }
            // products with the state and its gradient for this wave's 16 channels
            {
                const F3 fH = frag3(pH, PH, 16 * w + r16);
#pragma unroll
                for (int I = 0; I < NB; ++I) {
                    const int row = 16 * I + r16;
                    if constexpr (OEX)
                        X1[I] = mm3a(frag(pO, row), fH, X1[I]);
                    else
                        X1[I] = mm6(frag3(pO, PC, row), fH, X1[I]);
                    const u16x8 fUh = frag(pU, row), fUm = frag(pU + PC, row);
                    X3[I] = mmb(fUm, fH.h, X3[I]);
                    X3[I] = mmb(fUh, fH.m, X3[I]);
                    X3[I] = mmb(fUh, fH.h, X3[I]);
                }
            }
            {
                const F3 fdH = frag3(pdH, PH, 16 * w + r16);
#pragma unroll
                for (int I = 0; I < NB; ++I) X2[I] = mm6(frag3(pE, PC, 16 * I + r16), fdH, X2[I]);
            }
            // C x C products dO E^T and dUt E^T on the lower block tiles
#pragma unroll
            for (int sl = 0; sl < NYS; ++sl) {
                const int job = w + sl * NW;
                if (job < 2 * NY) {
                    int I, J;
                    lower_tile(job % NY, I, J);
                    const F3 fB = frag3(pE, PC, 16 * J + r16);
                    if (job >= NY)
                        Y[sl] = mm6(frag3(pU, PC, 16 * I + r16), fB, Y[sl]);
                    else if constexpr (OEX)
                        Y[sl] = mm3a(frag(pO, 16 * I + r16), fB, Y[sl]);
                    else
                        Y[sl] = mm6(frag3(pO, PC, 16 * I + r16), fB, Y[sl]);
                }
            }
        }
        // sum_n H dH per channel: lanes of one column quad differ in bits 2..5
#pragma unroll
        for (int z = 0; z < 4; ++z) {
            float t = gpart[z];
            t += __shfl_xor(t, 4);
            t += __shfl_xor(t, 8);
            t += __shfl_xor(t, 16);
            t += __shfl_xor(t, 32);
            gpart[z] = t;
        }
        // the row sums of dUt v: the eight threads of a row are consecutive lanes
#pragma unroll
        for (int j = 0; j < NZ; ++j) {
            float t = zpart[j];
            t += __shfl_xor(t, 1);
            t += __shfl_xor(t, 2);
            t += __shfl_xor(t, 4);
            zpart[j] = t;
        }
        // both handed to the channel's (row's) own thread through LDS after
        // the loop (sDb is rewritten with the whole dbeta term further on)
        lds_barrier();
        if (hp == 0) {
#pragma unroll
            for (int z = 0; z < 4; ++z) sDgam[4 * hcq + z] = gpart[z];
        }
        if ((tid & 7) == 0) {
#pragma unroll
            for (int j = 0; j < NZ; ++j) {
                const int e = tid + j * NT;
                if (e < 8 * C) sDb[e >> 3] = zpart[j];
            }
        }
        lds_barrier();
        if (tid < DK) gacc = sDgam[tid];
        if (tid < C) zacc = sDb[tid];
    } else {
        // One value slice of the records and inputs, requested into registers
        // while the previous slice is being used and written to LDS at the start
        // of its own turn.  Indices past the end are clamped for the loads (which
        // are then unconditional) and skipped for the LDS writes.
        constexpr int NHS = DK * VS / 4, NES = C * VS / 4, NOS = C * VS;
        constexpr int NH = (NHS + NT - 1) / NT, NE = (NES + NT - 1) / NT, NO = (NOS + NT - 1) / NT;
        struct Slice {
            f32x4 hh[NH], dh[NH], ee[NE], de[NE];
            float oo[NO], vv[NO];
        };
        auto load_slice = [&](Slice& x, int s) {
            const int v0 = s * VS;
    #pragma unroll
            for (int j = 0; j < NH; ++j) {
                const int e = min(tid + j * NT, NHS - 1);
                const int n = e / (DK / 4), c = 4 * (e % (DK / 4));
                const size_t o = R * a.r.rs + (size_t)(v0 + n) * DK + c;
                x.hh[j] = *reinterpret_cast<const f32x4*>(a.r.Hs + o);
                x.dh[j] = *reinterpret_cast<const f32x4*>(a.r.dH + o);
            }
    #pragma unroll
            for (int j = 0; j < NE; ++j) {
                const int e = min(tid + j * NT, NES - 1);
                const int n = e / (C / 4), i = 4 * (e % (C / 4));
                const size_t o = R * a.r.rs + (size_t)(v0 + n) * C + i;
                x.ee[j] = *reinterpret_cast<const f32x4*>(a.r.E + o);
                x.de[j] = *reinterpret_cast<const f32x4*>(a.r.dE + o);
            }
    #pragma unroll
            for (int j = 0; j < NO; ++j) {
                const int e = min(tid + j * NT, NOS - 1);
                const int i = clamp_row(e / VS, L), n = e % VS;
                x.oo[j] = io<IO>::load(dO + tok_v(a, b, t0 + i, h) * DV + v0 + n);
                x.vv[j] = io<IO>::load(v + tok_v(a, b, t0 + i, h) * DV + v0 + n);
            }
        };
        auto store_slice = [&](const Slice& x) {
    #pragma unroll
            for (int j = 0; j < NH; ++j) {
                const int e = tid + j * NT;
                if (e < NHS) {
                    const int n = e / (DK / 4), c = 4 * (e % (DK / 4));
                    *reinterpret_cast<f32x4*>(sH + n * LHT + c) = x.hh[j];
                    *reinterpret_cast<f32x4*>(sdH + n * LHT + c) = x.dh[j];
                }
            }
    #pragma unroll
            for (int j = 0; j < NE; ++j) {
                const int e = tid + j * NT;
                if (e < NES) {
                    const int n = e / (C / 4), i = 4 * (e % (C / 4));
                    *reinterpret_cast<f32x4*>(sE + n * LET + i) = x.ee[j];
    #pragma unroll
                    for (int z = 0; z < 4; ++z) sdE[n * LDE + i + z] = x.de[j][z];
                }
            }
    #pragma unroll
            for (int j = 0; j < NO; ++j) {
                const int e = tid + j * NT;
                if (e < NOS) {
                    const int i = e / VS, n = e % VS;
                    sdO[i * LV + n] = keep(x.oo[j], i, L);
                    sV[i * LV + n] = keep(x.vv[j], i, L);
                }
            }
        };

        Slice nx;
        load_slice(nx, 0);
        for (int s = 0; s < NS; ++s) {
            const int v0 = s * VS;
            lds_barrier();
            store_slice(nx);
            if (s + 1 < NS) load_slice(nx, s + 1);
            lds_barrier();
            // dUt = T^T dE (upper triangular: rows i take j >= 16 I), dv = beta dUt
            for (int job = w; job < NB * (VS / 16); job += NW) {
                const int I = job / (VS / 16), Vt = job % (VS / 16);
                f32x4 acc = zero4();
                for (int kk = 16 * I; kk < C; kk += 4)
                    acc = mma4(sT[(kk + q4) * LT + 16 * I + r16], sdE[(16 * Vt + r16) * LDE + kk + q4], acc);
    #pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const int i = 16 * I + 4 * q4 + ii, n = 16 * Vt + r16;
                    sdU[i * LV + n] = acc[ii];
                    if (i < L)
                        store_grad(a.dv, tok_v(a, b, t0 + i, h) * DV + v0 + n, sBeta[i] * acc[ii], a.gdt);
                }
            }
            lds_barrier();
            if (tid < C) {
                for (int n = 0; n < VS; ++n) zacc += sdU[tid * LV + n] * sV[tid * LV + n];
            }
            if (tid < DK) {
                for (int n = 0; n < VS; ++n) gacc += sH[n * LHT + tid] * sdH[n * LHT + tid];
            }
            // products with the state and its gradient for this wave's 16 channels
    #pragma unroll 2
            for (int kk = 0; kk < VS; kk += 4) {
                const float bH = sH[(kk + q4) * LHT + 16 * w + r16];
                const float bdH = sdH[(kk + q4) * LHT + 16 * w + r16];
    #pragma unroll
                for (int I = 0; I < NB; ++I) {
                    X1[I] = mma4(sdO[(16 * I + r16) * LV + kk + q4], bH, X1[I]);
                    X2[I] = mma4(sE[(kk + q4) * LET + 16 * I + r16], bdH, X2[I]);
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
    #pragma unroll 4
                    for (int kk = 0; kk < VS; kk += 4)
                        Y[sl] = mma4(A[(16 * I + r16) * LV + kk + q4], sE[(kk + q4) * LET + 16 * J + r16], Y[sl]);
                }
            }
        }
    }
    lds_barrier();

    // dAqk (inclusive lower) and beta_i dA_ij, dA = -(strict lower of dUt E^T);
    // the dbeta term sum_j dA_ij Ap_ij per tile goes to sPart
    float* sdAq = smem + S::oAq;
    float* sdAb = smem + S::oAb;
    if (tid < DK) sDgam[tid] = gacc;
    // the output phase's G, k and q (wave w: key channel c = 16 w + r16, rows
    // 16 I + 4 q4 + ii), requested before the staging below
    const int c = 16 * w + r16;
    float Gd[NB][4], kd[NB][4], qd[NB][4];
#pragma unroll
    for (int I = 0; I < NB; ++I) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int i = 16 * I + 4 * q4 + ii;
            Gd[I][ii] = a.r.G[R * a.r.rs + i * DK + c];
            const size_t o = tok_qk(a, b, t0 + clamp_row(i, L), hq) * DK + c;
            kd[I][ii] = io<IO>::load(k + o);
            qd[I][ii] = io<IO>::load(q + o);
        }
    }
    float apv[NYS][4];
#pragma unroll
    for (int sl = 0; sl < NYS; ++sl) {
        int I, J;
        lower_tile(min(w + sl * NW, 2 * NY - 1) % NY, I, J);
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
            apv[sl][ii] = a.r.Ap[R * a.r.rs + (16 * I + 4 * q4 + ii) * C + 16 * J + r16];
    }
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
                    const float part = row16_scan(dA * apv[sl][ii]);
                    if (r16 == 15) sPart[i][J] = part;
                    sdAb[i * LA + j] = sBeta[i] * dA;
                }
            }
        }
    }
    lds_barrier();
    if (tid < C) {
        float s = zacc;
        for (int J = 0; J < NB; ++J) s += sPart[tid][J];
        sDb[tid] = s;
    }

    // output phase: wave w owns key channels 16 w .. 16 w + 15; lane (r16, q4)
    // holds rows 16 I + 4 q4 + ii of channel 16 w + r16
    float* src0 = smem + S::oSrc + w * 2 * C * 16;
    float* src1 = src0 + C * 16;
    float* sRow = smem + S::oRow;
    float* sRowG = smem + S::oRowG;
#pragma unroll
    for (int I = 0; I < NB; ++I) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int i = 16 * I + 4 * q4 + ii;
            kd[I][ii] = keep(kd[I][ii], i, L);
            qd[I][ii] = keep(qd[I][ii], i, L);
        }
    }
    // sums over later tokens i >= j, reference row 16 J + 15.  A channel
    // flagged in block J (decay across the block beyond kBlockRange) leaves
    // block J out of the product and takes its terms exactly: lane (r16, q4)
    // gathers the block's 16 rows of its channel from the four lanes of its
    // column and sums exp(G_i - G_j) <= 1 pair by pair.
    f32x4 Pinv[NB];
#pragma unroll
    for (int J = NB - 1; J >= 0; --J) {
        const float Ge = __shfl(Gd[J][3], 48 + r16);
        const bool flJ = __shfl(Gd[J][0], r16) - Ge > kBlockRange;
#pragma unroll
        for (int I = J; I < NB; ++I) {
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int row = 16 * I + 4 * q4 + ii;
                const float f = (I == J && flJ) ? 0.f : ex(Gd[I][ii] - Ge);
                src0[row * 16 + r16] = kd[I][ii] * f;
                src1[row * 16 + r16] = a.scale * qd[I][ii] * f;
            }
        }
        wave_lds_sync();
        f32x4 acc = zero4();
        for (int kk = 16 * J; kk < C; kk += 4) {
            acc = mma4(sdAb[(kk + q4) * LA + 16 * J + r16], src0[(kk + q4) * 16 + r16], acc);
            acc = mma4(sdAq[(kk + q4) * LA + 16 * J + r16], src1[(kk + q4) * 16 + r16], acc);
        }
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) Pinv[J][ii] = ex(Ge - Gd[J][ii]) * acc[ii];
        if (__any(flJ)) {
            float Gx[16], kx[16], qx[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                Gx[t] = __shfl(Gd[J][t & 3], 16 * (t >> 2) + r16);
                kx[t] = __shfl(kd[J][t & 3], 16 * (t >> 2) + r16);
                qx[t] = __shfl(qd[J][t & 3], 16 * (t >> 2) + r16);
            }
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int jl = 4 * q4 + ii, j = 16 * J + jl;
                float sum = 0.f;
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    if (t >= jl) {
                        const int i = 16 * J + t;
                        sum += (sdAb[i * LA + j] * kx[t] + sdAq[i * LA + j] * a.scale * qx[t]) *
                               ex(Gx[t] - Gd[J][ii]);
                    }
                }
                if (flJ) Pinv[J][ii] += sum;
            }
        }
        wave_lds_sync();
    }

    // sums over earlier tokens j <= i (reference row 16 I), and with them each
    // 16-row block's dq, dk and dG (staged in src1 for the suffix sums); the
    // dbeta term -sum_c (dUt H^T)_ic k_ic e^G_ic goes to sRow
    const float Gl = __shfl(Gd[NB - 1][3], 48 + r16);
    const bool grouped = a.dqp != nullptr;
    float colPr = 0.f;
#pragma unroll
    for (int I = 0; I < NB; ++I) {
        const float Gs = __shfl(Gd[I][0], r16);
        const bool flI = Gs - __shfl(Gd[I][3], 48 + r16) > kBlockRange;
#pragma unroll
        for (int J = 0; J <= I; ++J) {
#pragma unroll
            for (int ii = 0; ii < 4; ++ii)
                src0[(16 * J + 4 * q4 + ii) * 16 + r16] =
                    (J == I && flI) ? 0.f : kd[J][ii] * ex(Gs - Gd[J][ii]);
        }
        wave_lds_sync();
        f32x4 ra = zero4(), rb = zero4();
        for (int kk = 0; kk < 16 * (I + 1); kk += 4) {
            const float bs = src0[(kk + q4) * 16 + r16];
            ra = mma4(sdAq[(16 * I + r16) * LA + kk + q4], bs, ra);
            rb = mma4(sdAb[(16 * I + r16) * LA + kk + q4], bs, rb);
        }
        // a channel flagged in block I: the block's own terms, exactly
        float xq[4] = {0.f, 0.f, 0.f, 0.f}, xb[4] = {0.f, 0.f, 0.f, 0.f};
        if (__any(flI)) {
            float Gx[16], kx[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                Gx[t] = __shfl(Gd[I][t & 3], 16 * (t >> 2) + r16);
                kx[t] = __shfl(kd[I][t & 3], 16 * (t >> 2) + r16);
            }
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int il = 4 * q4 + ii, i = 16 * I + il;
                float sq = 0.f, sb = 0.f;
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    if (t <= il) {
                        const float kj = kx[t] * ex(Gd[I][ii] - Gx[t]);
                        sq += sdAq[i * LA + 16 * I + t] * kj;
                        sb += sdAb[i * LA + 16 * I + t] * kj;
                    }
                }
                if (flI) {
                    xq[ii] = sq;
                    xb[ii] = sb;
                }
            }
        }
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const int i = 16 * I + 4 * q4 + ii;
            const float f = ex(Gd[I][ii] - Gs), eg = ex(Gd[I][ii]);
            const float dqv = a.scale * (eg * X1[I][ii] + f * ra[ii] + xq[ii]);
            const float pg = -sBeta[i] * eg * X3[I][ii] + f * rb[ii] + xb[ii];
            const float pr = ex(Gl - Gd[I][ii]) * X2[I][ii];
            const float dkv = pg + Pinv[I][ii] + pr;
            src1[i * 16 + r16] = kd[I][ii] * (pg - Pinv[I][ii] - pr) + qd[I][ii] * dqv;
            colPr += pr * kd[I][ii];
            const float x3 = row16_scan(X3[I][ii] * kd[I][ii] * eg);
            if (r16 == 15) sRow[w * C + i] = x3;
            if (i < L) {
                if (grouped) {
                    const size_t o = tok_v(a, b, t0 + i, h) * DK + c;
                    a.dqp[o] = dqv;
                    a.dkp[o] = dkv;
                } else {
                    const size_t o = tok_qk(a, b, t0 + i, hq) * DK + c;
                    store_grad(a.dq, o, dqv, a.gdt);
                    store_grad(a.dk, o, dkv, a.gdt);
                }
            }
        }
        wave_lds_sync();
    }
    colPr += __shfl_xor(colPr, 16);
    colPr += __shfl_xor(colPr, 32);
    if (q4 == 3) src1[(C - 1) * 16 + r16] += colPr + sDgam[c] * ex(Gl);
    wave_lds_sync();

    if (a.mode == KDA_GATE_CHANNEL) {
        // dg = suffix sums of dG over the rows of the chunk, per channel
        float seg[16];
        float tot = 0.f;
        if (16 * q4 < C) {
#pragma unroll
            for (int m = 15; m >= 0; --m) {
                tot += src1[(16 * q4 + m) * 16 + r16];
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
        // row sums of dG over this wave's 16 channels
        if (lane < C) {
            float x = 0.f;
#pragma unroll
            for (int cc = 0; cc < 16; ++cc) x += src1[lane * 16 + cc];
            sRowG[w * C + lane] = x;
        }
    }
    lds_barrier();
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
    const int units = (a.stab ? a.N : a.B) * a.H;
    const unsigned nrec = a.ctab ? (unsigned)a.H * (unsigned)a.Gmax : (unsigned)units * (unsigned)a.NC;
    if (nrec > 0) {
        hipLaunchKernelGGL((bwd_prep<C, DK, DV, IO>), dim3(nrec), dim3(prep_threads<C, DK, DV>()), 0, s,
                           a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const unsigned ur8 = (unsigned)((2 * units + 7) / 8) * 8;
    if constexpr (prep_split<C, DK, DV, IO>()) {
        // two value tiles per workgroup once one-tile workgroups would
        // outnumber the compute units (the records of a step are then loaded
        // once for both tiles)
        if (DV % 32 == 0 && (double)ur8 * (DV / 16) > (double)device_cus())
            hipLaunchKernelGGL((bwd_states_mc<C, DK, DV, DV % 32 == 0 ? 2 : 1>), dim3(ur8 * (DV / (DV % 32 == 0 ? 32 : 16))),
                               dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((bwd_states_mc<C, DK, DV, 1>), dim3(ur8 * (DV / 16)), dim3(256), 0, s, a);
    } else
        hipLaunchKernelGGL((bwd_states<C, DK, DV, IO>), dim3(ur8 * (DV / 16)),
                           dim3(64 * StateShape<C, DK>::NWS), 0, s, a);
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
    KDA_BWD_CASE(CC, 128, 16) KDA_BWD_CASE(CC, 128, 32) KDA_BWD_CASE(CC, 128, 64) KDA_BWD_CASE(CC, 128, 128) \
    KDA_BWD_CASE(CC, 16, 256) KDA_BWD_CASE(CC, 32, 256) KDA_BWD_CASE(CC, 64, 256) KDA_BWD_CASE(CC, 128, 256)

hipError_t launch_bwd_c16(const bwd::Args& a, int Dk, int Dv, kda_dtype dtype, hipStream_t s);
hipError_t launch_bwd_c32(const bwd::Args& a, int Dk, int Dv, kda_dtype dtype, hipStream_t s);
hipError_t launch_bwd_c64(const bwd::Args& a, int Dk, int Dv, kda_dtype dtype, hipStream_t s);

}  // namespace kda
