// quant.hip -- activation quantisation for the scaled matrix cores: bf16 rows
// to MX e4m3 elements with one UE8M0 scale per 32 consecutive elements (the
// pages' low-precision paths quantise activations before the matrix units:
// knivesysl README, "formats" and "key flags", fp6 weights with e4m3
// activations; Strata docs/INTEL.md, "The engine itself on Intel", an amax
// quantiser).  Per block: amax over the block, scale exponent X =
// floor(log2 amax) - 8 (e4m3's largest binade holds 448 = 1.75 * 2^8),
// clamped to [-127, 127], -127 for a block of zeros; each element x * 2^-X
// (exact) clamped to +-448 and rounded to the nearest e4m3 value by the
// hardware conversion.  Optionally the dequantised elements, value * 2^X,
// as bf16 (exact for activations in bf16's normal range).
#include "common.h"
#include "kernels.h"

namespace moeq {

// floor(log2 |v|) of a nonzero bf16 magnitude (bits without the sign)
__device__ inline int bf16_floor_log2(u32 m) {
    const int e = (int)(m >> 7);
    if (e != 0) return e - 127;
    return (31 - __builtin_clz(m)) - 133;           // subnormal: m * 2^-133
}

// One lane per block of 32: its 64 bytes in four 16-byte loads.
__global__ __launch_bounds__(256) void mx_quant_kernel(const uint16_t *__restrict__ x, int64_t nblocks,
                                                      uint8_t *__restrict__ codes, uint8_t *__restrict__ scales,
                                                      uint16_t *__restrict__ deq) {
    const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= nblocks) return;
    const uint4 *src = reinterpret_cast<const uint4 *>(x + 32 * b);
    uint4 q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = src[i];
    u32 w[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        w[4 * i] = q[i].x; w[4 * i + 1] = q[i].y; w[4 * i + 2] = q[i].z; w[4 * i + 3] = q[i].w;
    }
    u32 am = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) am = max(am, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
    int X = am ? bf16_floor_log2(am) - 8 : -127;
    X = min(127, max(-127, X));
    scales[b] = (uint8_t)(X + 127);
    u32 out[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        // elements 4i .. 4i+3 -> one dword of e4m3 codes (low byte = lowest element)
        float v[4];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const u32 p = w[2 * i + j];
            v[2 * j] = ldexpf(__builtin_bit_cast(float, p << 16), -X);
            v[2 * j + 1] = ldexpf(__builtin_bit_cast(float, p & 0xFFFF0000u), -X);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = __builtin_fminf(448.0f, __builtin_fmaxf(-448.0f, v[j]));
        u32 d = (u32)__builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
        d = (u32)__builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], (int)d, true);
        out[i] = d;
    }
    uint4 *dst = reinterpret_cast<uint4 *>(codes + 32 * b);
    dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
    dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
    if (deq) {
        const float sc = ldexpf(1.0f, X);
        u32 dq[16];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const f2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)out[i], false);
            const f2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)out[i], true);
            dq[2 * i] = (u32)f32_to_bf16_rne(lo.x * sc) | ((u32)f32_to_bf16_rne(lo.y * sc) << 16);
            dq[2 * i + 1] = (u32)f32_to_bf16_rne(hi.x * sc) | ((u32)f32_to_bf16_rne(hi.y * sc) << 16);
        }
        uint4 *dd = reinterpret_cast<uint4 *>(deq + 32 * b);
#pragma unroll
        for (int i = 0; i < 4; ++i) dd[i] = make_uint4(dq[4 * i], dq[4 * i + 1], dq[4 * i + 2], dq[4 * i + 3]);
    }
}

hipError_t launch_mx_quant(const uint16_t *x, int T, int H, uint8_t *codes, uint8_t *scales, uint16_t *deq,
                           hipStream_t s) {
    const int64_t nb = (int64_t)T * (H / 32);
    hipLaunchKernelGGL(mx_quant_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, s, x, nb, codes, scales, deq);
    return hipGetLastError();
}

}  // namespace moeq
