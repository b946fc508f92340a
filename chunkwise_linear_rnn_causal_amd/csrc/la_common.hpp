// la_common.hpp -- device helpers shared by the gfx950 kernels of liblinattn.
//
// MFMA operand layout used throughout (16x16 output tiles, 64-lane wavefront):
// lane l belongs to lane group g = l / 16 and column n = l % 16.
//   A operand (M x K): lane (g, n) supplies row m = n, E consecutive K-slots.
//   B operand (K x N): lane (g, n) supplies column n, the same E K-slots.
//   D (M x N, fp32):   lane (g, n) holds rows m = 4g + e (e = 0..3), column n.
// Which real contraction index sits in which K-slot is free as long as A and B
// agree; the kernels use that freedom to feed D tiles back as operands.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// 16 raw bytes as a native vector (copies of HIP's uint4 struct can become memory
// copies that keep a register array in scratch)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum Variant { V_PLAIN = 0, V_NORM = 1, V_DECAY = 2, V_GDN = 3, V_VDECAY = 4, V_KDA = 5 };

// MFMA traits per storage/operand type.
template <typename T> struct Mfma;

template <> struct Mfma<bf16> {
    static constexpr int E = 8;  // operand elements per lane (K = 32)
    using frag = bf16x8;
    __device__ static inline f32x4 mma(const frag &a, const frag &b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

template <> struct Mfma<f16> {
    static constexpr int E = 8;  // operand elements per lane (K = 32)
    using frag = f16x8;
    __device__ static inline f32x4 mma(const frag &a, const frag &b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};

// Tensor-core operand type for an input storage type. bf16 inputs are computed
// on fp16 operands: every bf16 value of magnitude in [2^-14, 65504] is exact in
// fp16, and the intermediates (state, scores, pseudo-values) then round to 11
// significant bits instead of 8, at the same MFMA rate.
template <typename TI> struct OpOf;
template <> struct OpOf<bf16> { using type = f16; };
template <> struct OpOf<float> { using type = float; };

template <> struct Mfma<float> {
    static constexpr int E = 1;  // K = 4
    using frag = float;
    __device__ static inline f32x4 mma(float a, float b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

template <typename T> __device__ inline T from_f32(float x);
template <> __device__ inline float from_f32<float>(float x) { return x; }
template <> __device__ inline bf16 from_f32<bf16>(float x) { return (bf16)x; }
template <> __device__ inline f16 from_f32<f16>(float x) { return (f16)x; }

template <typename T> __device__ inline float to_f32(T x);
template <> __device__ inline float to_f32<float>(float x) { return x; }
template <> __device__ inline float to_f32<bf16>(bf16 x) { return (float)x; }
template <> __device__ inline float to_f32<f16>(f16 x) { return (float)x; }

// E contiguous elements -> operand fragment (p must be E*sizeof(T) aligned).
template <typename T> __device__ inline typename Mfma<T>::frag ld_frag(const T *p);
template <> __device__ inline bf16x8 ld_frag<bf16>(const bf16 *p) {
    return *reinterpret_cast<const bf16x8 *>(p);
}
template <> __device__ inline f16x8 ld_frag<f16>(const f16 *p) {
    return *reinterpret_cast<const f16x8 *>(p);
}
template <> __device__ inline float ld_frag<float>(const float *p) { return *p; }

template <typename T> __device__ inline typename Mfma<T>::frag zero_frag();
template <> __device__ inline bf16x8 zero_frag<bf16>() {
    bf16x8 z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = (bf16)0.0f;
    return z;
}
template <> __device__ inline f16x8 zero_frag<f16>() {
    f16x8 z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = (f16)0.0f;
    return z;
}
template <> __device__ inline float zero_frag<float>() { return 0.0f; }

// Negated fragment (exact: flips the sign bit).
template <typename T> __device__ inline typename Mfma<T>::frag neg_frag(typename Mfma<T>::frag f);
template <> __device__ inline bf16x8 neg_frag<bf16>(bf16x8 f) {
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = -f[i];
    return f;
}
template <> __device__ inline f16x8 neg_frag<f16>(f16x8 f) {
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = -f[i];
    return f;
}
template <> __device__ inline float neg_frag<float>(float f) { return -f; }

// Four consecutive elements to / from memory (vectorised for both types).
template <typename T> struct Vec4;
template <> struct Vec4<bf16> { typedef bf16x4 type; };
template <> struct Vec4<f16> { typedef f16x4 type; };
template <> struct Vec4<float> { typedef f32x4 type; };

template <typename T> __device__ inline void st4(T *p, f32x4 x) {
    typename Vec4<T>::type v;
    v[0] = from_f32<T>(x[0]); v[1] = from_f32<T>(x[1]);
    v[2] = from_f32<T>(x[2]); v[3] = from_f32<T>(x[3]);
    *reinterpret_cast<typename Vec4<T>::type *>(p) = v;
}
template <typename T> __device__ inline f32x4 ld4(const T *p) {
    typename Vec4<T>::type v = *reinterpret_cast<const typename Vec4<T>::type *>(p);
    f32x4 r;
    r[0] = to_f32<T>(v[0]); r[1] = to_f32<T>(v[1]);
    r[2] = to_f32<T>(v[2]); r[3] = to_f32<T>(v[3]);
    return r;
}

// Eight consecutive elements held as fp32 (global or LDS).
template <typename T> __device__ inline void ld8(const T *p, float (&x)[8]) {
    f32x4 a = ld4<T>(p), b = ld4<T>(p + 4);
    x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3];
    x[4] = b[0]; x[5] = b[1]; x[6] = b[2]; x[7] = b[3];
}
template <typename T> __device__ inline void st8(T *p, const float (&x)[8]) {
    f32x4 a = {x[0], x[1], x[2], x[3]}, b = {x[4], x[5], x[6], x[7]};
    st4<T>(p, a);
    st4<T>(p + 4, b);
}

// Operand fragment of type TM read from memory holding type TI (converted).
template <typename TI, typename TM>
__device__ inline typename Mfma<TM>::frag ld_frag_as(const TI *p) {
    if constexpr (sizeof(TI) == sizeof(TM) && Mfma<TM>::E == 1) {
        return (typename Mfma<TM>::frag)(*p);
    } else {
        typename Mfma<TM>::frag f;
        float x[8];
        ld8<TI>(p, x);
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = from_f32<TM>(x[i]);
        return f;
    }
}

// Eight consecutive elements kept in their storage format (16 bytes for 2-byte
// types, 32 for fp32), so a prefetch holds raw registers until it is staged.
template <typename T> struct Raw8 { uint4 v[sizeof(T) / 2]; };

template <typename T> __device__ inline Raw8<T> ld_raw8(const T *p) {
    Raw8<T> r;
#pragma unroll
    for (int i = 0; i < (int)(sizeof(T) / 2); ++i) r.v[i] = reinterpret_cast<const uint4 *>(p)[i];
    return r;
}
template <typename T> __device__ inline Raw8<T> zero_raw8() {
    Raw8<T> r;
#pragma unroll
    for (int i = 0; i < (int)(sizeof(T) / 2); ++i) r.v[i] = make_uint4(0u, 0u, 0u, 0u);
    return r;
}
// Streaming (non-temporal) variants for data touched once.
typedef unsigned u32x4_nt __attribute__((ext_vector_type(4)));
template <typename T> __device__ inline Raw8<T> ld_raw8_nt(const T *p) {
    Raw8<T> r;
#pragma unroll
    for (int i = 0; i < (int)(sizeof(T) / 2); ++i) {
        const u32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt *>(p) + i);
        r.v[i] = make_uint4(v[0], v[1], v[2], v[3]);
    }
    return r;
}
template <typename T> __device__ inline void st8_nt(T *p, const float (&x)[8]) {
    typename Vec4<T>::type a, b;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        a[j] = from_f32<T>(x[j]);
        b[j] = from_f32<T>(x[4 + j]);
    }
    if constexpr (sizeof(T) == 2) {
        u32x4_nt v;
        v[0] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(a, a, 0, 1));
        v[1] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(a, a, 2, 3));
        v[2] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(b, b, 0, 1));
        v[3] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(b, b, 2, 3));
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4_nt *>(p));
    } else {
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4_nt, a), reinterpret_cast<u32x4_nt *>(p));
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4_nt, b), reinterpret_cast<u32x4_nt *>(p) + 1);
    }
}

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <typename T> __device__ inline void unpack8(const Raw8<T> &r, float (&x)[8]);
template <> __device__ inline void unpack8<bf16>(const Raw8<bf16> &r, float (&x)[8]) {
    const uint32_t w[4] = {r.v[0].x, r.v[0].y, r.v[0].z, r.v[0].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = bf16_lo(w[i]);
        x[2 * i + 1] = bf16_hi(w[i]);
    }
}
template <> __device__ inline void unpack8<f16>(const Raw8<f16> &r, float (&x)[8]) {
    const f16x8 h = *reinterpret_cast<const f16x8 *>(&r.v[0]);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (float)h[i];
}
template <> __device__ inline void unpack8<float>(const Raw8<float> &r, float (&x)[8]) {
    const uint32_t w[8] = {r.v[0].x, r.v[0].y, r.v[0].z, r.v[0].w, r.v[1].x, r.v[1].y, r.v[1].z, r.v[1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = __uint_as_float(w[i]);
}

// Transposed [rows][C] tile (token index innermost) with an XOR swizzle on
// 16-byte units: unit' = unit ^ f(row), f(row) = (row & 7) ^ 2 * ((row >> 3) & 3).
// Rows start on the same bank (the row pitch is a multiple of 128 bytes), so
//  - 16-byte operand reads by 8 lanes of consecutive rows hit 8 distinct units;
//  - 8-byte transposed writes by lanes of rows 8 apart (same row & 7) and
//    consecutive 4-token groups hit 16 distinct 8-byte slots.
// Reads of 8 aligned tokens (fp16) and writes of 4 aligned tokens stay
// contiguous because they never cross a unit.
template <int C, typename T> __device__ inline int tidx(int row, int s) {
    constexpr int EU = 16 / (int)sizeof(T);  // elements per 16-byte unit
    constexpr int NU = C / EU;               // units per row
    const int f = ((row & 7) ^ (2 * ((row >> 3) & 3))) & (NU - 1);
    return row * C + (((s / EU) ^ f) * EU) + (s % EU);
}

// Operand fragment X[k][col0 + n] for the K-slots {r0 .. r0+3, r0+16 .. r0+19}
// of this lane's group, from a row-major fp16 tile of pitch P, with two
// transpose loads. In a 16-lane group the transpose load hands lane i element e
// of the 8-byte row piece addressed by lane 4e + i/4, column i % 4; so lane j
// addresses row r + (j >> 2), columns col0 + 4 (j & 3).
template <int P>
__device__ inline f16x8 tr_frag(const f16 *X, int r0, int col0, int lane) {
    typedef short v4s __attribute__((ext_vector_type(4)));
    const int j = lane & 15;
    const f16 *p0 = X + (r0 + (j >> 2)) * P + col0 + 4 * (j & 3);
    const f16 *p1 = p0 + 16 * P;
    const v4s a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)(p0));
    const v4s b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)(p1));
    const f16x4 ha = __builtin_bit_cast(f16x4, a), hb = __builtin_bit_cast(f16x4, b);
    return f16x8{ha[0], ha[1], ha[2], ha[3], hb[0], hb[1], hb[2], hb[3]};
}

// fp16 fragment from two accumulator tiles (tile lo in slots 0..3, hi in 4..7),
// each element scaled by f.
__device__ inline f16x8 pack_tiles(const f32x4 &lo, const f32x4 &hi, float f) {
    return f16x8{(f16)(lo[0] * f), (f16)(lo[1] * f), (f16)(lo[2] * f), (f16)(lo[3] * f),
                 (f16)(hi[0] * f), (f16)(hi[1] * f), (f16)(hi[2] * f), (f16)(hi[3] * f)};
}

// DPP move of a float (row_mask / bank_mask select written rows / banks; lanes
// whose source is invalid or masked keep `old`).
template <int CTRL, int ROW_MASK = 0xf, int BANK_MASK = 0xf>
__device__ inline float dpp_f32(float old, float src) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                                 __builtin_bit_cast(int, src), CTRL,
                                                                 ROW_MASK, BANK_MASK, false));
}

// Inclusive prefix sum over the 64 lanes of a wave, with DPP only: row shifts
// by 1, 2, 4, 8 scan each 16-lane row, then row broadcasts of lanes 15 and 31
// carry the row totals forward (row_shr = 0x110 + n, row_bcast:15 = 0x142,
// row_bcast:31 = 0x143).
__device__ inline float wave_inclusive_sum(float x) {
    x += dpp_f32<0x111>(0.f, x);
    x += dpp_f32<0x112>(0.f, x);
    x += dpp_f32<0x114>(0.f, x);
    x += dpp_f32<0x118>(0.f, x);
    x += dpp_f32<0x142, 0xa>(0.f, x);
    x += dpp_f32<0x143, 0xc>(0.f, x);
    return x;
}

// Maximum over the 64 lanes of a wave of non-negative values, with DPP only
// (same row shifts and row broadcasts as wave_inclusive_sum; lane 63 ends with
// the maximum of all lanes). Returned wave-uniform.
__device__ inline float wave_max_nonneg(float x) {
    x = fmaxf(x, dpp_f32<0x111>(0.f, x));
    x = fmaxf(x, dpp_f32<0x112>(0.f, x));
    x = fmaxf(x, dpp_f32<0x114>(0.f, x));
    x = fmaxf(x, dpp_f32<0x118>(0.f, x));
    x = fmaxf(x, dpp_f32<0x142, 0xa>(0.f, x));
    x = fmaxf(x, dpp_f32<0x143, 0xc>(0.f, x));
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// Power-of-two operand scaling of a carried quantity (state, pseudo-values) of
// magnitude at most m: the shift s >= 0 with m * 2^-s < 2^8, so that the
// quantity can grow 256-fold before its fp16 operand overflows (s = 0 below 2^8:
// small values keep their fp16 representation). Scaling by 2^-s is exact.
__device__ inline int carry_shift(float m) {
    const int e = (int)((__float_as_uint(m) >> 23) & 0xffu);  // m < 2^(e - 126)
    return min(max(e - 134, 0), 120);
}
// 2^s for |s| <= 126 (exact).
__device__ inline float pow2i(int s) { return __uint_as_float((uint32_t)(127 + s) << 23); }

// XCD-aware block order: consecutive virtual ids go to the same XCD (blocks are
// handed to the 8 XCDs round-robin), so the d_v slices of one head share L2.
__device__ inline int xcd_virtual_block() {
    const int total = gridDim.x, bid = blockIdx.x;
    const int xcd = bid & 7, slot = bid >> 3;
    return xcd * (total >> 3) + min(xcd, total & 7) + slot;
}

}  // namespace la
