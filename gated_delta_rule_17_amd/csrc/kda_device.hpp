// Device-side building blocks shared by the KDA kernels (gfx950 / CDNA4).
//
// * bf16 <-> f32 conversion by bit manipulation (round-to-nearest-even).
// * A 16x16x32 matrix-core "tile step": D(16x16, f32) += A(16x32) * B(32x16).
//   For bf16 operands it is one v_mfma_f32_16x16x32_bf16; for f32 operands it
//   is eight v_mfma_f32_16x16x4_f32 over the same fragments.
//
// Fragment convention (one 64-lane wavefront, lane l, r = l % 16, g = l / 16):
//   A fragment: the 8 values A[r][8g .. 8g+7]
//   B fragment: the 8 values B[8g .. 8g+7][r], i.e. row r of B^T
//   accumulator: the 4 values D[4g .. 4g+3][r]
// So an operand stored row-major as [row][k] (A) or as [col][k] (B^T) is
// loaded by the same routine: lane l reads 8 consecutive k of row 16-tile
// row r.  Contracting the 32 k-indices in any fixed order is allowed; for the
// f32 path, step s of the eight 16x16x4 instructions contracts the indices
// {s, 8+s, 16+s, 24+s}, one per lane group, which keeps the same fragments.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

struct bf16_t {   // storage type of bfloat16 tensors: raw bits
    uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    // round-to-nearest-even (v_cvt_pk_bf16_f32 on gfx950)
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// ---- scalar load/store of the I/O storage types ---------------------------
template <typename T> struct io;
template <> struct io<float> {
    static __device__ __forceinline__ float load(const float* p) { return *p; }
    static __device__ __forceinline__ void store(float* p, float x) { *p = x; }
};
template <> struct io<bf16_t> {
    static __device__ __forceinline__ float load(const bf16_t* p) { return bf16_to_f32(p->bits); }
    static __device__ __forceinline__ void store(bf16_t* p, float x) { p->bits = f32_to_bf16(x); }
};

// ---- matrix-core fragments -------------------------------------------------
// Frag<T>: 8 consecutive k-values of one row, in operand type T.
template <typename T> struct Frag;

template <> struct Frag<bf16_t> {
    u16x8 v;
    __device__ __forceinline__ void zero() { v = (u16x8){0, 0, 0, 0, 0, 0, 0, 0}; }
    __device__ __forceinline__ void load(const bf16_t* p) { v = *reinterpret_cast<const u16x8*>(p); }
    __device__ __forceinline__ void store(bf16_t* p) const { *reinterpret_cast<u16x8*>(p) = v; }
    __device__ __forceinline__ float get(int i) const { return bf16_to_f32(v[i]); }
    __device__ __forceinline__ void set(int i, float x) { v[i] = f32_to_bf16(x); }
    // make the loaded value available here (the wait for its load goes here)
    __device__ __forceinline__ void settle() { asm volatile("" : "+v"(v)); }
};

template <> struct Frag<float> {
    f32x4 lo, hi;
    __device__ __forceinline__ void zero() { lo = (f32x4){0, 0, 0, 0}; hi = lo; }
    __device__ __forceinline__ void load(const float* p) {
        lo = *reinterpret_cast<const f32x4*>(p);
        hi = *reinterpret_cast<const f32x4*>(p + 4);
    }
    __device__ __forceinline__ void store(float* p) const {
        *reinterpret_cast<f32x4*>(p) = lo;
        *reinterpret_cast<f32x4*>(p + 4) = hi;
    }
    __device__ __forceinline__ float get(int i) const { return i < 4 ? lo[i] : hi[i - 4]; }
    __device__ __forceinline__ void set(int i, float x) { if (i < 4) lo[i] = x; else hi[i - 4] = x; }
    __device__ __forceinline__ void settle() { asm volatile("" : "+v"(lo), "+v"(hi)); }
};

// D += A * B over one 32-wide k step.
__device__ __forceinline__ f32x4 mma(const Frag<bf16_t>& a, const Frag<bf16_t>& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.v),
                                                   __builtin_bit_cast(bf16x8, b.v), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mma(const Frag<float>& a, const Frag<float>& b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[0], b.lo[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[1], b.lo[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[2], b.lo[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[3], b.lo[3], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[0], b.hi[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[1], b.hi[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[2], b.hi[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[3], b.hi[3], c, 0, 0, 0);
    return c;
}

// Plain f32 16x16x4 step: lane (r, g) supplies A[r][g] and B[g][r].
__device__ __forceinline__ f32x4 mma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Four consecutive values of an operand type, packed for one store.
template <typename T> struct Vec4;
template <> struct Vec4<float> {
    static __device__ __forceinline__ void store(float* p, f32x4 x) { *reinterpret_cast<f32x4*>(p) = x; }
    static __device__ __forceinline__ f32x4 load(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
};
template <> struct Vec4<bf16_t> {
    static __device__ __forceinline__ void store(bf16_t* p, f32x4 x) {
        u16x4 u = {f32_to_bf16(x[0]), f32_to_bf16(x[1]), f32_to_bf16(x[2]), f32_to_bf16(x[3])};
        *reinterpret_cast<u16x4*>(p) = u;
    }
    static __device__ __forceinline__ f32x4 load(const bf16_t* p) {
        u16x4 u = *reinterpret_cast<const u16x4*>(p);
        return (f32x4){bf16_to_f32(u[0]), bf16_to_f32(u[1]), bf16_to_f32(u[2]), bf16_to_f32(u[3])};
    }
};

__device__ __forceinline__ f32x4 zero4() { return (f32x4){0.f, 0.f, 0.f, 0.f}; }

// ---- precise operands --------------------------------------------------------
// A float32 value x is carried as the bf16 pair (hi, lo) with hi = bf16(x) and
// lo = bf16(x - hi), which keeps about 16 significant bits.  A product of two
// such operands is formed from three bf16 matrix-core steps,
//   hi*hi + hi*lo + lo*hi,
// dropping only lo*lo (relative size 2^-16).  For float32 operand type the
// pair degenerates to the plain float32 value and one float32 step.
template <typename T> struct PFrag;
template <> struct PFrag<bf16_t> {
    Frag<bf16_t> h, l;
    __device__ __forceinline__ void load(const bf16_t* ph, const bf16_t* pl) { h.load(ph); l.load(pl); }
    __device__ __forceinline__ void from_f32(const float* x) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint16_t hb = f32_to_bf16(x[i]);
            h.v[i] = hb;
            l.v[i] = f32_to_bf16(x[i] - bf16_to_f32(hb));
        }
    }
};
template <> struct PFrag<float> {
    Frag<float> h;
    __device__ __forceinline__ void load(const float* ph, const float*) { h.load(ph); }
    __device__ __forceinline__ void from_f32(const float* x) {
        h.lo = (f32x4){x[0], x[1], x[2], x[3]};
        h.hi = (f32x4){x[4], x[5], x[6], x[7]};
    }
};

__device__ __forceinline__ f32x4 mma3(const PFrag<bf16_t>& a, const PFrag<bf16_t>& b, f32x4 c) {
    c = mma(a.l, b.h, c);
    c = mma(a.h, b.l, c);
    return mma(a.h, b.h, c);
}
__device__ __forceinline__ f32x4 mma3(const PFrag<float>& a, const PFrag<float>& b, f32x4 c) {
    return mma(a.h, b.h, c);
}

// D += A B over a 16-wide k given as four values per lane: lane (r, g)
// supplies A[r][4g .. 4g+3] (read from memory) and B[4g .. 4g+3][r], which is
// the layout of a 16x16 accumulator, so an accumulator serves directly as the
// right operand.  bf16: the precise product hi*hi + hi*lo + lo*hi of the
// pairs on v_mfma_f32_16x16x16_bf16; float32: four 16x16x4 steps, step u
// contracting the indices k = 4g + u.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mma16_p(const bf16_t* ah, const bf16_t* al, f32x4 b, f32x4 c) {
    const s16x4 a_h = *reinterpret_cast<const s16x4*>(ah);
    const s16x4 a_l = *reinterpret_cast<const s16x4*>(al);
    s16x4 b_h, b_l;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const uint16_t hb = f32_to_bf16(b[u]);
        b_h[u] = (short)hb;
        b_l[u] = (short)f32_to_bf16(b[u] - bf16_to_f32(hb));
    }
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a_l, b_h, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a_h, b_l, c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a_h, b_h, c, 0, 0, 0);
}
// A 16x16 accumulator (or any four values per lane in that layout) as a
// right operand of the 16-wide products: plain and hi/lo bf16 parts.
struct B16 {
    s16x4 h, l;
    __device__ __forceinline__ static B16 from(f32x4 x) {
        B16 r;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint16_t hb = f32_to_bf16(x[u]);
            r.h[u] = (short)hb;
            r.l[u] = (short)f32_to_bf16(x[u] - bf16_to_f32(hb));
        }
        return r;
    }
    __device__ __forceinline__ static B16 plain(f32x4 x) {
        B16 r;
#pragma unroll
        for (int u = 0; u < 4; ++u) r.h[u] = (short)f32_to_bf16(x[u]);
        r.l = r.h;
        return r;
    }
};
// precise: A pair from memory times a pre-split right operand
__device__ __forceinline__ f32x4 mma16_p(const bf16_t* ah, const bf16_t* al, const B16& b, f32x4 c) {
    const s16x4 a_h = *reinterpret_cast<const s16x4*>(ah);
    const s16x4 a_l = *reinterpret_cast<const s16x4*>(al);
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a_l, b.h, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a_h, b.l, c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a_h, b.h, c, 0, 0, 0);
}
// the same with the left operand already in registers
__device__ __forceinline__ f32x4 mma16v(s16x4 a, s16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16v_p(s16x4 ah, s16x4 al, const B16& b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, b.h, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, b.l, c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, b.h, c, 0, 0, 0);
}
// plain: one bf16 product (hi parts only)
__device__ __forceinline__ f32x4 mma16(const bf16_t* a, const B16& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(*reinterpret_cast<const s16x4*>(a), b.h, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16_p(const float* a, const float*, f32x4 b, f32x4 c) {
    const f32x4 av = *reinterpret_cast<const f32x4*>(a);
#pragma unroll
    for (int u = 0; u < 4; ++u) c = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u], b[u], c, 0, 0, 0);
    return c;
}

// Plain operand times precise operand: a * (b.hi + b.lo), and the mirror.
__device__ __forceinline__ f32x4 mma2(const Frag<bf16_t>& a, const PFrag<bf16_t>& b, f32x4 c) {
    c = mma(a, b.l, c);
    return mma(a, b.h, c);
}
__device__ __forceinline__ f32x4 mma2(const Frag<float>& a, const PFrag<float>& b, f32x4 c) {
    return mma(a, b.h, c);
}
__device__ __forceinline__ f32x4 mma2(const PFrag<bf16_t>& a, const Frag<bf16_t>& b, f32x4 c) {
    c = mma(a.l, b, c);
    return mma(a.h, b, c);
}
__device__ __forceinline__ f32x4 mma2(const PFrag<float>& a, const Frag<float>& b, f32x4 c) {
    return mma(a.h, b, c);
}

// Pair of arrays holding the hi and lo parts of a precise operand (lo is
// unused, and may be null, for float32).
template <typename T> struct PArr {
    T* h; T* l;
    __device__ __forceinline__ PFrag<T> frag(int idx) const { PFrag<T> f; f.load(h + idx, l + idx); return f; }
    // four consecutive values as float32 (hi + lo)
    __device__ __forceinline__ f32x4 load4(int idx) const {
        if constexpr (sizeof(T) == 2) return Vec4<T>::load(h + idx) + Vec4<T>::load(l + idx);
        else return Vec4<T>::load(h + idx);
    }
};

__device__ __forceinline__ void store_p(const PArr<bf16_t>& a, int idx, float x) {
    const uint16_t hb = f32_to_bf16(x);
    a.h[idx].bits = hb;
    a.l[idx].bits = f32_to_bf16(x - bf16_to_f32(hb));
}
__device__ __forceinline__ void store_p(const PArr<float>& a, int idx, float x) { a.h[idx] = x; }

__device__ __forceinline__ void store4_p(const PArr<bf16_t>& a, int idx, f32x4 x) {
    f32x4 hv, lv;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const uint16_t hb = f32_to_bf16(x[u]);
        hv[u] = bf16_to_f32(hb);
        lv[u] = x[u] - hv[u];
    }
    Vec4<bf16_t>::store(a.h + idx, hv);
    Vec4<bf16_t>::store(a.l + idx, lv);
}
__device__ __forceinline__ void store4_p(const PArr<float>& a, int idx, f32x4 x) {
    Vec4<float>::store(a.h + idx, x);
}

}  // namespace kda
