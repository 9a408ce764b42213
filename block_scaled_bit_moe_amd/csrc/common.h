// common.h -- device building blocks shared by the gfx950 kernels.
//
// Formats (knivesysl README, "formats"; colibri README, "DeepSeek V4" and its
// model notes):
//   FMT 1: e2m1 codes, two per byte (low nibble = even element), one fp8 e4m3
//          scale per 16 weights;
//   FMT 2: e2m3 codes as a little-endian 6-bit stream, one UE8M0 scale per 128;
//   FMT 3: e2m1 codes, one UE8M0 scale per 32 (MXFP4);
//   FMT 4: two's-complement int4 codes (packed as e2m1), one fp16 scale per 64
//          (two bytes, low byte first);
//   FMT 5: e2m3 codes, one fp8 e4m3 scale per 16.
// Everything here works on "units" of 32 consecutive weights of one row:
//   four-bit codes: 16 code bytes; six-bit codes: 24 code bytes; plus the
//   unit's scale bits (two e4m3 bytes for the per-16 formats, the byte of its
//   UE8M0 block, or the fp16 of its int4 group).
// A unit decodes to 16 bf16x2 registers (exact: every e2m1, e2m3 and int4
// value has at most 4 significant bits) which v_dot2c_f32_bf16 multiplies with
// 16 bf16x2 of the activation, accumulating in fp32; the block scale is
// applied once per block with an fp32 FMA.
#pragma once

#include <hip/hip_runtime.h>
#include <type_traits>
#include <stdint.h>

#include "kernels.h"

namespace moeq {

typedef uint32_t u32;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(6))) u32 u32x6_t;
typedef __attribute__((ext_vector_type(32))) __bf16 bf16x32_t;
typedef __attribute__((ext_vector_type(2))) float f2_t;

constexpr int FMT_E2M1 = 1;     // e2m1 + e4m3 per 16
constexpr int FMT_E2M3 = 2;     // e2m3 + UE8M0 per 128
constexpr int FMT_MXFP4 = 3;    // e2m1 + UE8M0 per 32
constexpr int FMT_INT4 = 4;     // int4 + fp16 per 64
constexpr int FMT_E2M3S = 5;    // e2m3 + e4m3 per 16
constexpr int WAVE = 64;

// Scale kinds
constexpr int SC_E4M3 = 0, SC_UE8M0 = 1, SC_FP16 = 2;
// Code kinds
constexpr int CODE_E2M1 = 0, CODE_E2M3 = 1, CODE_INT4 = 2;

template <int FMT> struct Fmt {
    static_assert(FMT >= 1 && FMT <= 5, "format");
    static constexpr int CODE = (FMT == FMT_E2M1 || FMT == FMT_MXFP4) ? CODE_E2M1 : (FMT == FMT_INT4 ? CODE_INT4 : CODE_E2M3);
    static constexpr bool SIX = CODE == CODE_E2M3;                 // six-bit codes
    static constexpr int UNIT_CODE_BYTES = SIX ? 24 : 16;
    static constexpr int BLOCK = FMT == FMT_E2M3 ? 128 : FMT == FMT_MXFP4 ? 32 : FMT == FMT_INT4 ? 64 : 16;
    static constexpr int SCALE = (FMT == FMT_E2M1 || FMT == FMT_E2M3S) ? SC_E4M3 : (FMT == FMT_INT4 ? SC_FP16 : SC_UE8M0);
    static constexpr bool TWO_SCALES = BLOCK == 16;                // two blocks per unit
    __host__ __device__ static inline int64_t code_row_bytes(int64_t cols) { return SIX ? cols * 3 / 4 : cols / 2; }
    __host__ __device__ static inline int64_t scale_row_bytes(int64_t cols) {
        return SCALE == SC_FP16 ? 2 * (cols / BLOCK) : cols / BLOCK;
    }
};

// ----------------------------------------------------------------------------
// Value tables, built on the device from the bit fields.
// A minifloat with `eb` exponent bits of bias `bias`, `mb` mantissa bits,
// subnormals at exponent field 0: the float value of code c (sign at bit eb+mb).
__device__ __host__ inline float minifloat_value(u32 c, int eb, int mb, int bias) {
    u32 m = c & ((1u << mb) - 1u);
    u32 e = (c >> mb) & ((1u << eb) - 1u);
    u32 s = (c >> (mb + eb)) & 1u;
    float mag = (e == 0) ? ldexpf((float)m / (float)(1u << mb), 1 - bias)
                         : ldexpf(1.0f + (float)m / (float)(1u << mb), (int)e - bias);
    return s ? -mag : mag;
}

__device__ inline u32 bf16_bits_exact(float f) {   // f has <= 8 significant bits
    return __builtin_bit_cast(u32, f) >> 16;
}

// LDS table sizes (in u32 entries)
constexpr int LUT_E2M1_PAIR = 256;     // byte -> bf16x2 (low nibble in the low half)
constexpr int LUT_E2M3_PAIR = 4096;    // 12 bits (two codes) -> bf16x2
constexpr int LUT_SCALE = 256;         // e4m3 or UE8M0 byte -> fp32

struct Luts {
    u32 *pair;      // e2m1 or e2m3 pair table
    float *scale;   // e4m3 or UE8M0
};

// Fill the tables (call by the whole block, then __syncthreads()).  The pair
// table holds two decoded codes per entry (e2m1 and int4: one byte; e2m3:
// twelve bits); the scale table the format's scale byte (fp16 scales are
// converted arithmetically and need none).
template <int FMT>
__device__ inline void build_luts(const Luts &L, int tid, int nthreads, bool need_pair) {
    using F = Fmt<FMT>;
    if (need_pair) {
        if constexpr (F::CODE == CODE_E2M3) {
            for (int p = tid; p < LUT_E2M3_PAIR; p += nthreads) {
                u32 lo = bf16_bits_exact(minifloat_value(p & 63, 2, 3, 1));
                u32 hi = bf16_bits_exact(minifloat_value(p >> 6, 2, 3, 1));
                L.pair[p] = lo | (hi << 16);
            }
        } else {
            for (int b = tid; b < LUT_E2M1_PAIR; b += nthreads) {
                u32 lo, hi;
                if constexpr (F::CODE == CODE_E2M1) {
                    lo = bf16_bits_exact(minifloat_value(b & 15, 2, 1, 1));
                    hi = bf16_bits_exact(minifloat_value(b >> 4, 2, 1, 1));
                } else {   // int4: the nibble as a signed 4-bit integer
                    lo = bf16_bits_exact((float)(((int)((u32)b << 28)) >> 28));
                    hi = bf16_bits_exact((float)(((int)((u32)b << 24)) >> 28));
                }
                L.pair[b] = lo | (hi << 16);
            }
        }
    }
    for (int b = tid; b < LUT_SCALE; b += nthreads) {
        if constexpr (F::SCALE == SC_E4M3) L.scale[b] = ((b & 0x7F) == 0x7F) ? __builtin_nanf("") : minifloat_value(b, 4, 3, 7);
        else L.scale[b] = (b == 255) ? __builtin_nanf("") : ldexpf(1.0f, b - 127);
    }
}

// ----------------------------------------------------------------------------
// Raw unit loads
template <bool SIX> struct UnitCodes;
template <> struct UnitCodes<false> {
    uint4 c;        // 16 code bytes = 32 weights
};
template <> struct UnitCodes<true> {
    uint2 c0, c1, c2;   // 24 code bytes = 32 weights
};
// s: the unit's scale bits -- two e4m3 bytes in bits 0..15 (per-16 formats),
// its UE8M0 block's byte, or its int4 group's fp16 bits
template <int FMT> struct Unit : UnitCodes<Fmt<FMT>::SIX> { u32 s; };

__device__ inline uint4 ldg16(const uint8_t *p) { return *reinterpret_cast<const uint4 *>(p); }
__device__ inline uint2 ldg8(const uint8_t *p) { return *reinterpret_cast<const uint2 *>(p); }

// Load unit u of a row (codes/scales point at the row's first byte).
template <int FMT>
__device__ inline void load_unit(Unit<FMT> &U, const uint8_t *codes, const uint8_t *scales, int u) {
    using F = Fmt<FMT>;
    if constexpr (!F::SIX) {
        U.c = ldg16(codes + (int64_t)u * 16);
    } else {
        const uint8_t *p = codes + (int64_t)u * 24;
        U.c0 = ldg8(p);
        U.c1 = ldg8(p + 8);
        U.c2 = ldg8(p + 16);
    }
    if constexpr (F::TWO_SCALES) U.s = *reinterpret_cast<const uint16_t *>(scales + 2 * u);
    else if constexpr (F::SCALE == SC_FP16) U.s = *reinterpret_cast<const uint16_t *>(scales + 2 * (u >> 1));
    else U.s = scales[u / (F::BLOCK / 32)];
}

// int4 pair from a nibble pair: both nibbles sign-extended, converted exactly
__device__ inline u32 int4_pair_bf16(u32 d, int shift) {
    const int lo = ((int)(d << (28 - shift))) >> 28, hi = ((int)(d << (24 - shift))) >> 28;
    const bf16x2_t b = bf16x2_t{(__bf16)(float)lo, (__bf16)(float)hi};
    return __builtin_bit_cast(u32, b);
}

// Decode a unit into 16 bf16x2 words (pair i = weights 2i, 2i+1; low half = even).
template <int FMT, int DEC>
__device__ inline void decode_unit(const Unit<FMT> &U, const Luts &L, u32 w[16]) {
    using F = Fmt<FMT>;
    if constexpr (!F::SIX) {
        const u32 d[4] = {U.c.x, U.c.y, U.c.z, U.c.w};
        if constexpr (DEC == DEC_HW && F::CODE == CODE_E2M1) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                w[4 * i + 0] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], 1.0f, 0));
                w[4 * i + 1] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], 1.0f, 1));
                w[4 * i + 2] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], 1.0f, 2));
                w[4 * i + 3] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], 1.0f, 3));
            }
        } else if constexpr (DEC == DEC_HW) {   // int4: sign extension and exact integer conversion
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int b = 0; b < 4; ++b) w[4 * i + b] = int4_pair_bf16(d[i], 8 * b);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int b = 0; b < 4; ++b) w[4 * i + b] = L.pair[(d[i] >> (8 * b)) & 0xFF];
            }
        }
    } else {
        const u32 d[6] = {U.c0.x, U.c0.y, U.c1.x, U.c1.y, U.c2.x, U.c2.y};
        if constexpr (DEC == DEC_HW) {
            u32x6_t v;
            v[0] = d[0]; v[1] = d[1]; v[2] = d[2]; v[3] = d[3]; v[4] = d[4]; v[5] = d[5];
            bf16x32_t r = __builtin_amdgcn_cvt_scalef32_pk32_bf16_fp6(v, 1.0f);
            typedef __attribute__((ext_vector_type(16))) u32 u32x16_t;
            u32x16_t rr = __builtin_bit_cast(u32x16_t, r);
#pragma unroll
            for (int i = 0; i < 16; ++i) w[i] = rr[i];
        } else {
#pragma unroll
            for (int p = 0; p < 16; ++p) {
                const int bit = 12 * p, dw = bit >> 5, off = bit & 31;
                u32 f;
                if (off + 12 <= 32) f = (d[dw] >> off) & 0xFFFu;
                else f = __builtin_amdgcn_alignbit(d[dw + 1], d[dw], off) & 0xFFFu;
                w[p] = L.pair[f];
            }
        }
    }
}

__device__ inline float dot2(u32 a, u32 b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// acc += dot(unit weights, x) with the block scale(s) applied once per block.
// Two interleaved partial sums per block keep the dot2 dependency chains short.
template <int FMT>
__device__ inline float unit_dot(const u32 w[16], const u32 x[16], float s0, float s1, float acc) {
    if constexpr (Fmt<FMT>::TWO_SCALES) {
        float a0 = 0.f, b0 = 0.f, a1 = 0.f, b1 = 0.f;
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
            a0 = dot2(w[i], x[i], a0);
            b0 = dot2(w[i + 1], x[i + 1], b0);
            a1 = dot2(w[8 + i], x[8 + i], a1);
            b1 = dot2(w[9 + i], x[9 + i], b1);
        }
        acc = __builtin_fmaf(s0, a0 + b0, acc);
        return __builtin_fmaf(s1, a1 + b1, acc);
    } else {
        float a = 0.f, b = 0.f, c = 0.f, d = 0.f;
#pragma unroll
        for (int i = 0; i < 16; i += 4) {
            a = dot2(w[i], x[i], a);
            b = dot2(w[i + 1], x[i + 1], b);
            c = dot2(w[i + 2], x[i + 2], c);
            d = dot2(w[i + 3], x[i + 3], d);
        }
        (void)s1;
        return __builtin_fmaf(s0, (a + b) + (c + d), acc);
    }
}

// Same with the activation carried as bf16 hi + lo (x = hi + lo to ~16 bits):
// both parts meet the same decoded weights and the same block scale.
template <int FMT>
__device__ inline float unit_dot_split(const u32 w[16], const u32 xh[16], const u32 xl[16], float s0, float s1,
                                       float acc) {
    if constexpr (Fmt<FMT>::TWO_SCALES) {
        float a0 = 0.f, b0 = 0.f, a1 = 0.f, b1 = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a0 = dot2(w[i], xh[i], a0);
            b0 = dot2(w[i], xl[i], b0);
            a1 = dot2(w[8 + i], xh[8 + i], a1);
            b1 = dot2(w[8 + i], xl[8 + i], b1);
        }
        acc = __builtin_fmaf(s0, a0 + b0, acc);
        return __builtin_fmaf(s1, a1 + b1, acc);
    } else {
        float a = 0.f, b = 0.f, c = 0.f, d = 0.f;
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
            a = dot2(w[i], xh[i], a);
            b = dot2(w[i], xl[i], b);
            c = dot2(w[i + 1], xh[i + 1], c);
            d = dot2(w[i + 1], xl[i + 1], d);
        }
        (void)s1;
        return __builtin_fmaf(s0, (a + b) + (c + d), acc);
    }
}

// The unit's block scale(s) as fp32: e4m3 and UE8M0 bytes through the LDS
// table, fp16 by the exact hardware conversion.
template <int FMT>
__device__ inline void unit_scales(const Unit<FMT> &U, const Luts &L, float &s0, float &s1) {
    using F = Fmt<FMT>;
    if constexpr (F::TWO_SCALES) {
        s0 = L.scale[U.s & 0xFF];
        s1 = L.scale[(U.s >> 8) & 0xFF];
    } else if constexpr (F::SCALE == SC_FP16) {
        s0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(U.s & 0xFFFF));
        s1 = 0.f;
    } else {
        s0 = L.scale[U.s & 0xFF];
        s1 = 0.f;
    }
}

// ----------------------------------------------------------------------------
// Wave reductions with DPP (no LDS traffic, a few cycles per step).  Sum over
// aligned groups of G lanes; the same butterfly runs in every group, so the
// order of the additions is fixed.  For G <= 16 every lane of the group holds
// the sum; for G = 32 / 64 the sum is valid in the group's first lane only
// (the rows of 16 are added there in ascending order with readlane).
template <int CTRL>
__device__ inline float dpp_mov(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

__device__ inline float group_sum_dpp(float v, int G) {
    if (G >= 2) v += dpp_mov<0xB1>(v);    // quad_perm [1,0,3,2]
    if (G >= 4) v += dpp_mov<0x4E>(v);    // quad_perm [2,3,0,1]
    if (G >= 8) v += dpp_mov<0x141>(v);   // row_half_mirror
    if (G >= 16) v += dpp_mov<0x140>(v);  // row_mirror
    if (G == 32) {
        const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
        const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
        const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
        const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
        v = ((threadIdx.x & 63) < 32) ? r0 + r1 : r2 + r3;
    } else if (G == 64) {
        const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
        const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
        const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
        const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
        v = ((r0 + r1) + r2) + r3;
    }
    return v;
}

// ----------------------------------------------------------------------------
// Routing helpers.  Order key of an fp32 logit: a larger float gets a larger
// key, +0 and -0 get the same key, NaN gets 1 (below every number); 0 is left
// for "no expert".
__device__ inline u32 logit_key(float f) {
    u32 b = __builtin_bit_cast(u32, f);
    if ((b & 0x7FFFFFFFu) > 0x7F800000u) return 1u;   // NaN
    if (b == 0x80000000u) b = 0u;                      // -0 == +0
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ inline float logit_of_key(u32 k) {
    if (k <= 1u) return __builtin_nanf("");
    const u32 b = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __builtin_bit_cast(float, b);
}

template <int CTRL, int ROWMASK = 0xF>
__device__ inline u32 dpp_u32(u32 old, u32 v) {
    return (u32)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROWMASK, 0xF, false);
}

// max over the 64 lanes, returned uniform: four in-row DPP stages
// (each lane's source is always valid, so the move folds into the max), then
// the four row results combined on the scalar unit
template <int CTRL>
__device__ inline u32 dpp_mov_u32(u32 v) {
    return (u32)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
__device__ inline u32 wave_max_u32(u32 v) {
    v = max(v, dpp_mov_u32<0xB1>(v));         // quad_perm [1,0,3,2]
    v = max(v, dpp_mov_u32<0x4E>(v));         // quad_perm [2,3,0,1]
    v = max(v, dpp_mov_u32<0x141>(v));        // row_half_mirror
    v = max(v, dpp_mov_u32<0x140>(v));        // row_mirror
    const u32 r0 = (u32)__builtin_amdgcn_readlane((int)v, 0);
    const u32 r1 = (u32)__builtin_amdgcn_readlane((int)v, 16);
    const u32 r2 = (u32)__builtin_amdgcn_readlane((int)v, 32);
    const u32 r3 = (u32)__builtin_amdgcn_readlane((int)v, 48);
    return max(max(r0, r1), max(r2, r3));
}


// One wave routes one token: the k best experts in rank order and their
// softmax weights over the k picks (Strata docs/INTEL.md, "The engine itself on
// Intel": router_top10, for any k).
//
// Every expert gets a unique 64-bit key: the order key of its logit in the
// high half and the complement of its index in the low half, so a larger key
// means a larger logit, or the same logit and a lower index — the ranking
// rule itself, with no tie left to break.  Lane l holds experts
// l*PER_LANE .. l*PER_LANE + PER_LANE - 1 (contiguous loads) and sorts its keys
// once (bitonic network, descending).  Each of the k rounds takes the wave
// maximum of the lanes' first keys (two 32-bit DPP maxima: the logit half,
// then the index half among the holders of that logit); the lane whose first
// key it is drops it.  The winner's index is in the key itself.  Lanes 0 .. k-1 end with
// (idx, w) of rank = lane; other lanes return idx -1.
template <int PER_LANE>
__device__ inline void route_load_logits(const float *__restrict__ logits, int E, int lane, float (&lg)[PER_LANE]) {
#pragma unroll
    for (int j = 0; j < PER_LANE; ++j) lg[j] = logits[min(lane * PER_LANE + j, E - 1)];   // all loads in flight
}

// Per-lane bitonic sort of PER_LANE unique 64-bit keys, descending.
template <int PER_LANE>
__device__ inline void sort_keys_desc(uint64_t (&key)[PER_LANE]) {
#pragma unroll
    for (int sz = 2; sz <= PER_LANE; sz <<= 1)
#pragma unroll
        for (int j = sz >> 1; j > 0; j >>= 1)
#pragma unroll
            for (int i = 0; i < PER_LANE; ++i) {
                const int l = i ^ j;
                if (l > i) {
                    const bool desc = (i & sz) == 0;
                    const bool sw = desc ? (key[l] > key[i]) : (key[l] < key[i]);
                    const uint64_t a = key[i], b = key[l];
                    key[i] = sw ? b : a;
                    key[l] = sw ? a : b;
                }
            }
}

// Unique routing key of expert e with logit v: the order key of the logit in
// the high half, the complement of the index in the low half (0: no expert).
__device__ inline uint64_t expert_key(float v, int e, bool valid) {
    return ((uint64_t)(valid ? logit_key(v) : 0u) << 32) | (u32)~(u32)e;
}

// k rounds over per-lane lists sorted descending: round r takes the wave-wide
// largest first key (its logit half, then among the lanes holding that logit
// its index half) and the lane holding it drops it.  Lane r ends with the key
// of rank r (lanes >= k: 0).
template <int PER_LANE>
__device__ inline uint64_t topk_rounds(uint64_t (&key)[PER_LANE], int k, int lane) {
    uint64_t mine = 0;
    for (int r = 0; r < k; ++r) {
        const u32 hv = (u32)(key[0] >> 32), hl = (u32)key[0];
        const u32 mv = wave_max_u32(hv);
        const uint64_t holders = __ballot(hv == mv);
        u32 ml;
        if (__popcll(holders) == 1)      // the usual case: one lane holds that logit
            ml = (u32)__builtin_amdgcn_readlane((int)hl, __ffsll((long long)holders) - 1);
        else
            ml = wave_max_u32(hv == mv ? hl : 0u);
        const bool win = hv == mv && hl == ml;
#pragma unroll
        for (int j = 0; j + 1 < PER_LANE; ++j) key[j] = win ? key[j + 1] : key[j];
        if (win) key[PER_LANE - 1] = 0u;
        if (lane == r) mine = ((uint64_t)mv << 32) | ml;
    }
    return mine;
}

// Lanes 0 .. k-1 hold the keys of ranks 0 .. k-1: their experts and the
// softmax over the k picked logits in fp32, exp(l_r - l_0) summed in rank order.
__device__ inline void weights_from_ranked(uint64_t mine, int k, int lane, int &my_idx, float &my_w) {
    const float my_l = logit_of_key((u32)(mine >> 32));
    const float l0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, my_l), 0));
    my_idx = (lane < k) ? (int)~(u32)mine : -1;
    const float ex = (lane < k) ? expf(my_l - l0) : 0.f;
    float z = 0.f;
    for (int r = 0; r < k; ++r) z += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, ex), r));
    my_w = (lane < k) ? ex / z : 0.f;
}

template <int PER_LANE>
__device__ inline void route_from_logits(const float (&lg)[PER_LANE], int E, int k, int lane, int &my_idx,
                                         float &my_w) {
    uint64_t key[PER_LANE];
#pragma unroll
    for (int j = 0; j < PER_LANE; ++j) {
        const int e = lane * PER_LANE + j;
        key[j] = expert_key(lg[j], e, e < E);
    }
    sort_keys_desc<PER_LANE>(key);
    const uint64_t mine = topk_rounds<PER_LANE>(key, k, lane);
    weights_from_ranked(mine, k, lane, my_idx, my_w);
}

template <int PER_LANE>
__device__ inline void route_one_token_wave(const float *__restrict__ logits, int E, int k, int lane, int &my_idx,
                                            float &my_w) {
    float lg[PER_LANE];
    route_load_logits<PER_LANE>(logits, E, lane, lg);
    route_from_logits<PER_LANE>(lg, E, k, lane, my_idx, my_w);
}

__device__ inline float silu_f32(float g) { return g / (1.0f + expf(-g)); }

__device__ inline float bf16_to_f32(uint16_t b) { return __builtin_bit_cast(float, (u32)b << 16); }

__device__ inline uint16_t f32_to_bf16_rne(float f) {
    u32 u = __builtin_bit_cast(u32, f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);   // quiet NaN
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

}  // namespace moeq
