// mfma_unit.h -- one weight unit (32 consecutive weights of a row and their
// block scale) as the B operand of the bf16 matrix instructions
// (v_mfma_f32_16x16x32_bf16), the block scale folded in exactly.  Shared by
// the grouped GEMMs of the many-token layer and the batched dense GEMV.
#pragma once

#include "common.h"

namespace moeq {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) u32 u32x4_t;

// int4 weights times their fp16 group scale need up to 14 significant bits, so
// they enter the matrix cores as two bf16 parts, w = hi + lo exactly
template <int FMT> constexpr bool pf_split_w() { return Fmt<FMT>::SCALE == SC_FP16; }

// Decode one unit, block scale included, into the B operands of the four MFMA
// steps of a K step (step s takes weights 8s .. 8s+7 of the unit).
//  e2m1 + e4m3 and e2m3 + e4m3: codes -> fp32, times the scale of their block
//    of 16 (exact: a code value has at most 4 significant bits and an e4m3
//    scale 4, and the product stays inside bf16's range), packed to bf16;
//  e2m3 + UE8M0 and e2m1 + UE8M0: the conversion applies the power-of-two
//    scale itself (it takes the scale's exponent field, which is all a UE8M0
//    scale has): exact while code value times scale stays inside bf16's range;
//  int4 + fp16: w = code * scale is exact in fp32 but needs up to 14 bits, so
//    it is split into bf16 hi = RNE(w) and lo = w - hi (exact, at most 7 bits)
//    and the matrix cores take both (b and bl).
__device__ inline u32 pf_pack2(float a, float b) { return __builtin_bit_cast(u32, bf16x2_t{(__bf16)a, (__bf16)b}); }

template <int FMT>
__device__ inline void pf_unit_to_b(const Unit<FMT> &U, const float *s_scale, bf16x8_t (&b)[4], bf16x8_t (&bl)[4]) {
    using F = Fmt<FMT>;
    if constexpr (FMT == FMT_E2M1) {
        const float s0 = s_scale[U.s & 0xFF], s1 = s_scale[(U.s >> 8) & 0xFF];
        const u32 d[4] = {U.c.x, U.c.y, U.c.z, U.c.w};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const float sc = s < 2 ? s0 : s1;
            const f2_t f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d[s], 1.0f, 0);
            const f2_t f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d[s], 1.0f, 1);
            const f2_t f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d[s], 1.0f, 2);
            const f2_t f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d[s], 1.0f, 3);
            u32x4_t v;
            v[0] = pf_pack2(f0.x * sc, f0.y * sc);
            v[1] = pf_pack2(f1.x * sc, f1.y * sc);
            v[2] = pf_pack2(f2.x * sc, f2.y * sc);
            v[3] = pf_pack2(f3.x * sc, f3.y * sc);
            b[s] = __builtin_bit_cast(bf16x8_t, v);
        }
    } else if constexpr (FMT == FMT_MXFP4) {
        const float sc = __builtin_bit_cast(float, (U.s & 0xFFu) << 23);
        const u32 d[4] = {U.c.x, U.c.y, U.c.z, U.c.w};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            u32x4_t v;
            v[0] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[s], sc, 0));
            v[1] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[s], sc, 1));
            v[2] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[s], sc, 2));
            v[3] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[s], sc, 3));
            b[s] = __builtin_bit_cast(bf16x8_t, v);
        }
    } else if constexpr (FMT == FMT_INT4) {
        const float sc = (float)__builtin_bit_cast(_Float16, (uint16_t)(U.s & 0xFFFF));
        const u32 d[4] = {U.c.x, U.c.y, U.c.z, U.c.w};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            u32x4_t vh, vl;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float w0 = (float)(((int)(d[s] << (28 - 8 * q))) >> 28) * sc;
                const float w1 = (float)(((int)(d[s] << (24 - 8 * q))) >> 28) * sc;
                const u32 h = pf_pack2(w0, w1);
                vh[q] = h;
                vl[q] = pf_pack2(w0 - __builtin_bit_cast(float, h << 16), w1 - __builtin_bit_cast(float, h & 0xFFFF0000u));
            }
            b[s] = __builtin_bit_cast(bf16x8_t, vh);
            bl[s] = __builtin_bit_cast(bf16x8_t, vl);
        }
    } else if constexpr (FMT == FMT_E2M3S) {
        u32x6_t v;
        v[0] = U.c0.x; v[1] = U.c0.y; v[2] = U.c1.x; v[3] = U.c1.y; v[4] = U.c2.x; v[5] = U.c2.y;
        typedef __attribute__((ext_vector_type(32))) float f32x32_t;
        const f32x32_t f = __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(v, 1.0f);
        const float s0 = s_scale[U.s & 0xFF], s1 = s_scale[(U.s >> 8) & 0xFF];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const float sc = s < 2 ? s0 : s1;
            u32x4_t q4;
#pragma unroll
            for (int q = 0; q < 4; ++q) q4[q] = pf_pack2(f[8 * s + 2 * q] * sc, f[8 * s + 2 * q + 1] * sc);
            b[s] = __builtin_bit_cast(bf16x8_t, q4);
        }
    } else {
        static_assert(FMT == FMT_E2M3, "format");
        u32x6_t v;
        v[0] = U.c0.x; v[1] = U.c0.y; v[2] = U.c1.x; v[3] = U.c1.y; v[4] = U.c2.x; v[5] = U.c2.y;
        const float sc = __builtin_bit_cast(float, (U.s & 0xFFu) << 23);
        const bf16x32_t r = __builtin_amdgcn_cvt_scalef32_pk32_bf16_fp6(v, sc);
        typedef __attribute__((ext_vector_type(16))) u32 u32x16_t;
        const u32x16_t rr = __builtin_bit_cast(u32x16_t, r);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            u32x4_t q;
            q[0] = rr[4 * s]; q[1] = rr[4 * s + 1]; q[2] = rr[4 * s + 2]; q[3] = rr[4 * s + 3];
            b[s] = __builtin_bit_cast(bf16x8_t, q);
        }
    }
    (void)F::SIX;
}

template <int FMT>
__device__ inline void pf_zero_unit(Unit<FMT> &U) {
    if constexpr (!Fmt<FMT>::SIX) {
        U.c = make_uint4(0u, 0u, 0u, 0u);
    } else {
        U.c0 = make_uint2(0u, 0u);
        U.c1 = U.c0;
        U.c2 = U.c0;
    }
    U.s = 0u;
}

// An empty asm that "rewrites" a unit's registers: placed where the unit is
// consumed (after an explicit vmcnt wait, or where the compiler's own wait
// for it belongs), it keeps the compiler from hoisting uses of the loaded
// values (such as masking a scale byte) to an earlier point, where its
// waitcnt pass would also wait for every younger load.
template <int FMT>
__device__ inline void pf_pin_unit(Unit<FMT> &U) {
    if constexpr (!Fmt<FMT>::SIX)
        asm volatile("" : "+v"(U.c.x), "+v"(U.c.y), "+v"(U.c.z), "+v"(U.c.w), "+v"(U.s));
    else
        asm volatile("" : "+v"(U.c0.x), "+v"(U.c0.y), "+v"(U.c1.x), "+v"(U.c1.y), "+v"(U.c2.x), "+v"(U.c2.y),
                     "+v"(U.s));
}

}  // namespace moeq
