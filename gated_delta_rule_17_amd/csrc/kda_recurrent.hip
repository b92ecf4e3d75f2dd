// Recurrent (token-by-token) KDA forward: the decode kernel.
//
// GeekNews #31925, section "Fused recurrent kernel for decode": the state of
// one sequence and head stays on chip while the tokens are processed in
// order, each token doing decay -> prediction (a reduction over the key
// dimension) -> residual -> rank-1 write -> read (a second reduction).
//
// MI355X mapping: one workgroup (up to 512 threads for a decode step, 256 for
// several tokens per sequence; see RecShape) owns the whole state of
// one (batch, head), so every wave instruction reads and writes whole
// contiguous rows (a slab split of the columns over two workgroups, with
// half-rows per instruction, measured 5% slower).  The transposed state
// H = S^T (Dk x Dv, float32) is loaded ONCE from HBM into registers with
// 16-byte loads -- thread (rg, cx) holds columns 4cx..4cx+3 in rows rg,
// rg+RG, rg+2RG, ... -- and written back ONCE at the end.  The first token's
// inputs are requested before the state, so they arrive first.  Per token:
//   Ht   = Diag(exp g_t) H                          (rows scaled)
//   vhat = Ht^T k,  r = Ht^T q~,  kq = k . q~       (one pass over the rows)
//   e    = beta (v - vhat)
//   H    = Ht + k e^T
//   o    = H^T q~ = r + e * kq                      (no second pass needed)
// The partial sums are reduced across the rows a wavefront holds with lane
// shuffles, then across wavefronts through LDS.
#include <atomic>

#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {

// x[l] + x[l ^ 32] in every lane l, on the vector unit: v_permlane32_swap
// with x as both operands returns the lower half's values in the first
// result and the upper half's in the second, in every lane (the same sums as
// an xor-32 shuffle, without the LDS round trip)
__device__ __forceinline__ float add_halves(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Threads per workgroup: up to 512 for a decode step (the state streamed at
// the HBM rate); up to 256 for several tokens per sequence, whose token steps
// are a serial chain: with one wave per SIMD and twice the rows per thread, a
// step issues fewer vector instructions per SIMD (the cross-wave sums of the
// reductions shrink with the number of waves).
template <int DK, int DV, bool MULTI>
struct RecShape {
    static constexpr int DVT = DV > 128 ? 128 : DV; // columns per workgroup
    static constexpr int NCT = DV / DVT;            // workgroups per (b, h)
    static constexpr int NTMAX = MULTI ? 256 : 512;
    static constexpr int NT = (DK * DVT / 4 < NTMAX) ? DK * DVT / 4 : NTMAX;  // threads
    static constexpr int CX = DVT / 4;       // threads across the slab (float4 each)
    static constexpr int RG = NT / CX;       // row groups
    static constexpr int RPT = DK / RG;      // rows per thread
    static constexpr int NW = NT / 64;       // wavefronts
    static_assert(NT % 64 == 0 && RPT >= 1 && RG * RPT == DK && CX <= 64, "shape");
    static_assert(NT >= DK && NT >= DVT, "every key channel and value column has a thread");
};

// MULTI: sequences of more than one token (the next token's inputs are
// prefetched during the current one); without it every sequence has at most
// one token (a decode step), and the state's rows are used as they arrive.
template <int DK, int DV, typename IO, typename OUT, bool MULTI>
__global__ void __launch_bounds__((RecShape<DK, DV, MULTI>::NT))
recurrent_kernel(const IO* __restrict__ q, const IO* __restrict__ k, const IO* __restrict__ v,
                 const float* __restrict__ g, const float* __restrict__ beta,
                 float* __restrict__ state, OUT* __restrict__ o,
                 int T, int H, int HQ, float scale, int mode, const int* __restrict__ cu, int pro)
{
    using S = RecShape<DK, DV, MULTI>;
    const int bh = blockIdx.x / S::NCT;
    const int c0 = (blockIdx.x - bh * S::NCT) * S::DVT;   // first column of the slab
    const int b = bh / H, h = bh - (bh / H) * H;
    // the tokens of this sequence: [b*T, b*T + T) of a dense batch, or
    // [cu[b], cu[b+1]) of a packed one (T is then the packed token count;
    // the offsets are clamped into [0, T] and the end to at least the start,
    // so no access leaves the buffers whatever they hold)
    size_t tok0 = (size_t)b * T;
    int Tn = T;
    if (cu) {
        const int s0 = min(max(cu[b], 0), T);
        const int s1 = min(max(cu[b + 1], s0), T);
        tok0 = (size_t)s0;
        Tn = s1 - s0;
    }
    const int tid = threadIdx.x;
    const int cx = tid % S::CX, rg = tid / S::CX;
    const int lane = tid & 63, wave = tid >> 6;

    // per key channel (alpha, k, scale * q, 0): one 16-byte read per row; two
    // buffers, token t in buffer t & 1, so that token t+1's inputs are
    // committed while token t's may still be read
    __shared__ __align__(16) f32x4 akq[2][DK];
    __shared__ float sv[2][S::DVT];
    // per wavefront and column group the 11 partial sums, padded to 12 so
    // that they move as three 16-byte accesses
    __shared__ __align__(16) float red[S::NW > 1 ? S::NW : 1][S::CX][12];

    float* st = state + (size_t)bh * DK * DV + c0;
    // (value head h reads query/key head h / (H / HQ): grouped value heads)
    const int hq = h / (H / HQ);
    // The inputs of one token as this thread reads them (thread c < DK owns key
    // channel c, thread j < DVT value column j; every thread reads beta).  The
    // loads are unconditional, from clamped indices, so that no branch joins
    // loaded registers; commit() moves them to LDS.  Token t+1's inputs are
    // requested while token t is computed.
    // (raw storage values: converted only in commit(), so that nothing waits
    // for the loads before then)
    struct TokIn { IO k, q, v; float g, b; };
    const int ck = tid < DK ? tid : DK - 1, cv = tid < S::DVT ? tid : S::DVT - 1;
    // gate address of a row: g[row][h][ck] (channel), g[row][h] (scalar); without
    // a gate beta stands in (a valid address; the value is unused)
    const float* gbase = mode == KDA_GATE_NONE ? beta : g;
    const size_t gstride = mode == KDA_GATE_CHANNEL ? (size_t)H * DK : (size_t)H;
    const size_t goff = mode == KDA_GATE_CHANNEL ? (size_t)h * DK + ck : (size_t)h;
    auto fetch = [&](size_t row, TokIn& x) {
        const size_t tok = row * H + h, tkq = row * HQ + hq;
        x.k = k[tkq * DK + ck];
        x.q = q[tkq * DK + ck];
        x.g = gbase[row * gstride + goff];
        x.v = v[tok * DV + c0 + cv];
        x.b = beta[tok];
    };
    auto commit = [&](const TokIn& x, int buf) {
        if (tid < DK) {
            // the retention alpha = exp(g), or sigmoid(a) from a pre-activation
            float a = 1.f;
            if (mode != KDA_GATE_NONE)
                a = (pro & KDA_GATE_LOGSIGMOID) ? 1.f / (1.f + expf(-x.g)) : expf(x.g);
            akq[buf][tid] = (f32x4){a, io<IO>::load(&x.k), io<IO>::load(&x.q) * scale, 0.f};
        }
        if (tid < S::DVT) sv[buf][tid] = io<IO>::load(&x.v);
    };
    // the first token's inputs, requested before the state so that they arrive first
    TokIn cur;
    if (Tn > 0) fetch(tok0, cur);
    f32x4 hr[S::RPT];
#pragma unroll
    for (int i = 0; i < S::RPT; ++i)
        hr[i] = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4*>(st + (size_t)(rg + S::RG * i) * DV + 4 * cx));

    if (Tn > 0) commit(cur, 0);
    float bcur = cur.b;
    // one token: decay, the two reductions over the rows, correction, rank-1
    // write and read (inputs in LDS, beta in bcur)
    auto token = [&](size_t tok, int buf) {
            f32x4 ak = zero4(), aq = zero4();
            float kq = 0.f, kk = 0.f, qq = 0.f;
    #pragma unroll
            for (int i = 0; i < S::RPT; ++i) {
                const f32x4 row = akq[buf][rg + S::RG * i];
                const float a = row[0], kr = row[1], qr = row[2];
                hr[i] *= a;
                ak += hr[i] * kr;
                aq += hr[i] * qr;
                kq += kr * qr;
            }
            if (pro & KDA_NORMALIZE_QK) {   // the norms' partial sums
    #pragma unroll
                for (int i = 0; i < S::RPT; ++i) {
                    const f32x4 row = akq[buf][rg + S::RG * i];
                    kk += row[1] * row[1];
                    qq += row[2] * row[2];
                }
            }
            // reduce over the row groups held by this wavefront
    #pragma unroll
            for (int off = S::CX; off < 32; off <<= 1) {
    #pragma unroll
                for (int u = 0; u < 4; ++u) {
                    ak[u] += __shfl_xor(ak[u], off);
                    aq[u] += __shfl_xor(aq[u], off);
                }
                kq += __shfl_xor(kq, off);
                kk += __shfl_xor(kk, off);
                qq += __shfl_xor(qq, off);
            }
            if constexpr (S::CX < 64) {
    #pragma unroll
                for (int u = 0; u < 4; ++u) {
                    ak[u] = add_halves(ak[u]);
                    aq[u] = add_halves(aq[u]);
                }
                kq = add_halves(kq);
                kk = add_halves(kk);
                qq = add_halves(qq);
            }
            if constexpr (S::NW > 1) {
                if (lane < S::CX) {
                    f32x4* rp = reinterpret_cast<f32x4*>(&red[wave][cx][0]);
                    rp[0] = ak;
                    rp[1] = aq;
                    rp[2] = (f32x4){kq, kk, qq, 0.f};
                }
                __syncthreads();
                // every thread needs the prediction sums (for e); only the
                // threads that write o (row group 0) need the query sums and
                // k.q, and k.k and q.q matter only for the normalisation
                ak = zero4();
    #pragma unroll
                for (int w = 0; w < S::NW; ++w) ak += reinterpret_cast<const f32x4*>(&red[w][cx][0])[0];
                if (rg == 0 || (pro & KDA_NORMALIZE_QK)) {
                    f32x4 sc = zero4();
    #pragma unroll
                    for (int w = 0; w < S::NW; ++w) sc += reinterpret_cast<const f32x4*>(&red[w][cx][0])[2];
                    kq = sc[0]; kk = sc[1]; qq = sc[2];
                }
                if (rg == 0) {
                    aq = zero4();
    #pragma unroll
                    for (int w = 0; w < S::NW; ++w) aq += reinterpret_cast<const f32x4*>(&red[w][cx][0])[1];
                }
            }
            // L2-normalised q and k: every product with them is linear, so the
            // norms are applied to the reduced sums (akq holds scale * q)
            float fk = 1.f, fq = 1.f;
            if (pro & KDA_NORMALIZE_QK) {
                fk = rsqrtf(kk + kNormEps);
                fq = scale != 0.f ? rsqrtf(qq / (scale * scale) + kNormEps) : 1.f;
                ak *= fk;
                aq *= fq;
                kq *= fk * fq;
            }
            float bt = bcur;
            if (pro & KDA_BETA_SIGMOID) bt = 1.f / (1.f + expf(-bt));
            f32x4 e;
    #pragma unroll
            for (int u = 0; u < 4; ++u) e[u] = bt * (sv[buf][4 * cx + u] - ak[u]);
            const f32x4 ek = e * fk;
    #pragma unroll
            for (int i = 0; i < S::RPT; ++i) hr[i] += akq[buf][rg + S::RG * i][1] * ek;
            if (rg == 0) {
                Vec4<OUT>::store(o + tok * DV + c0 + 4 * cx, aq + e * kq);
            }
    };
    if constexpr (!MULTI) {
        // a decode step: the state's rows are used as they arrive
        if (Tn == 1) {
            __syncthreads();
            token(tok0 * H + h, 0);
        }
    } else {
        // three tokens in flight: slot j holds the inputs of a token requested
        // three token steps before it is committed (one step is shorter than a
        // load's round trip).  The slots rotate statically, with no register
        // copy of a load in flight; past the end the last token is requested
        // again.  They are requested after the state's rows, so no wait for
        // those rows counts them, and loads complete in order, so committing
        // one slot does not wait for the two requested after it.
        TokIn s0, s1, s2;
        if (Tn > 0) {
            fetch(tok0 + min(1, Tn - 1), s0);
            fetch(tok0 + min(2, Tn - 1), s1);
            fetch(tok0 + min(3, Tn - 1), s2);
        }
        // One barrier per token besides the reduction's: token t+1's inputs
        // go to the other buffer, whose last reader (token t-1) every thread
        // has left at token t's reduction barrier, and the partial sums are
        // rewritten only after the next token's first barrier.
        auto step = [&](int t, TokIn& slot) {
            __syncthreads();   // token t's inputs are in LDS
            token((tok0 + t) * H + h, t & 1);
            commit(slot, (t + 1) & 1);   // token t+1
            bcur = slot.b;
            fetch(tok0 + min(t + 4, Tn - 1), slot);
        };
        for (int t = 0; t < Tn; t += 3) {
            step(t, s0);
            if (t + 1 < Tn) step(t + 1, s1);
            if (t + 2 < Tn) step(t + 2, s2);
        }
    }
#pragma unroll
    for (int i = 0; i < S::RPT; ++i)
        __builtin_nontemporal_store(
            hr[i], reinterpret_cast<f32x4*>(st + (size_t)(rg + S::RG * i) * DV + 4 * cx));
}


// Dynamic LDS the decode launch reserves so that at most two of its
// workgroups share a compute unit: with three (the registers would allow it)
// the state stream measured 7% slower (190 us against 177 us for the B256 H32
// d128 step).  Two fit when each workgroup takes 2/5 of the unit's LDS.
static size_t decode_lds_reserve(size_t static_bytes)
{
    static std::atomic<long long> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    const int slot = dev < 64 ? dev : 63;
    long long per_cu = cache[slot].load(std::memory_order_relaxed);
    if (per_cu <= 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess ||
            v <= 0)
            v = 65536;
        per_cu = v;
        cache[slot].store(per_cu, std::memory_order_relaxed);
    }
    const size_t want = (size_t)per_cu * 2 / 5;
    return want > static_bytes ? want - static_bytes : 0;
}

template <int DK, int DV, typename IO, bool MULTI>
static hipError_t launch_rec2(const RecArgs& a, hipStream_t s)
{
    using S = RecShape<DK, DV, MULTI>;
    size_t dyn = 0;
    if constexpr (!MULTI) {
        // the kernel's own LDS: akq and sv (two buffers each) and the reduction array
        const size_t static_bytes = 2 * (4 * DK + S::DVT) * 4 + (S::NW > 1 ? S::NW : 1) * S::CX * 12 * 4;
        dyn = decode_lds_reserve(static_bytes);
    }
    if (a.o_dtype == KDA_F32)
        hipLaunchKernelGGL((recurrent_kernel<DK, DV, IO, float, MULTI>), dim3(a.B * a.H * S::NCT), dim3(S::NT), dyn, s,
                           (const IO*)a.q, (const IO*)a.k, (const IO*)a.v, a.g, a.beta, a.state,
                           (float*)a.o, a.T, a.H, a.Hq, a.scale, (int)a.mode, a.cu, a.prologue);
    else
        hipLaunchKernelGGL((recurrent_kernel<DK, DV, IO, bf16_t, MULTI>), dim3(a.B * a.H * S::NCT), dim3(S::NT), dyn, s,
                           (const IO*)a.q, (const IO*)a.k, (const IO*)a.v, a.g, a.beta, a.state,
                           (bf16_t*)a.o, a.T, a.H, a.Hq, a.scale, (int)a.mode, a.cu, a.prologue);
    return hipGetLastError();
}

template <int DK, int DV, typename IO>
static hipError_t launch_rec(const RecArgs& a, hipStream_t s)
{
    // one token per sequence (a dense T = 1 call): the decode kernel
    if (a.cu == nullptr && a.T == 1) return launch_rec2<DK, DV, IO, false>(a, s);
    return launch_rec2<DK, DV, IO, true>(a, s);
}

template <int DK, typename IO>
static hipError_t dispatch_dv(const RecArgs& a, hipStream_t s)
{
    switch (a.Dv) {
        case 16: return launch_rec<DK, 16, IO>(a, s);
        case 32: return launch_rec<DK, 32, IO>(a, s);
        case 64: return launch_rec<DK, 64, IO>(a, s);
        case 128: return launch_rec<DK, 128, IO>(a, s);
        case 256: return launch_rec<DK, 256, IO>(a, s);
    }
    return hipErrorInvalidValue;
}

template <typename IO>
static hipError_t dispatch_dk(const RecArgs& a, hipStream_t s)
{
    switch (a.Dk) {
        case 16: return dispatch_dv<16, IO>(a, s);
        case 32: return dispatch_dv<32, IO>(a, s);
        case 64: return dispatch_dv<64, IO>(a, s);
        case 128: return dispatch_dv<128, IO>(a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_recurrent(const RecArgs& a, hipStream_t s)
{
    if (a.dtype == KDA_BF16) return dispatch_dk<bf16_t>(a, s);
    return dispatch_dk<float>(a, s);
}

}  // namespace kda
