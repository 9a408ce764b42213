// gemv.hip -- dense_gemv_q: y[b] = W x[b] for a block-scaled W and B <= 8 bf16
// tokens that share every decoded weight (knivesysl README, "formats": the fp6
// e2m3 projections with a power-of-two scale per 128; Strata docs/INTEL.md,
// "Decode round 2": aligned 16-byte weight loads).  Bandwidth-bound: each
// weight byte is read once from HBM per pass of MT tokens.
#include "kernels.h"
#include "rowdot.h"

namespace moeq {

template <int FMT, int DEC, int Q, int MT, int R>
__global__ __launch_bounds__(256) void gemv_kernel(const uint8_t *__restrict__ codes,
                                                   const uint8_t *__restrict__ scales, int rows, int cols,
                                                   const uint16_t *__restrict__ x, int B, void *__restrict__ y,
                                                   int out_f32) {
    constexpr int PAIR = (DEC == DEC_LUT) ? (FMT == FMT_E2M1 ? LUT_E2M1_PAIR : LUT_E2M3_PAIR) : 1;
    __shared__ u32 s_pair[PAIR];
    __shared__ float s_scale[LUT_SCALE];
    const Luts L{s_pair, s_scale};
    build_luts<FMT>(L, threadIdx.x, blockDim.x, DEC == DEC_LUT);
    __syncthreads();

    const int U = cols / 32;
    const int LPR = lanes_per_row(U);
    const int lane = threadIdx.x & 63, lr = lane & (LPR - 1), rsub = lane / LPR, RPW = WAVE / LPR;
    const int64_t crb = Fmt<FMT>::code_row_bytes(cols), srb = Fmt<FMT>::scale_row_bytes(cols);
    const int nw = gridDim.x * (blockDim.x / WAVE);
    const int gw = blockIdx.x * (blockDim.x / WAVE) + (threadIdx.x >> 6);
    const int ngroups = (rows + RPW - 1) / RPW;

    for (int t0 = 0; t0 < B; t0 += MT) {
        u32 xr[Q][MT][16];
        const uint16_t *xp[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) xp[t] = (t0 + t < B) ? x + (int64_t)(t0 + t) * cols : nullptr;
        load_x_units<Q, MT>(xr, xp, U, lr, LPR);

        for (int g0 = gw; g0 < ngroups; g0 += nw * R) {
            const uint8_t *crow[R], *srow[R];
            int row[R];
            bool valid[R];
#pragma unroll
            for (int b = 0; b < R; ++b) {
                const int grp = g0 + b * nw;
                row[b] = grp * RPW + rsub;
                valid[b] = (grp < ngroups) && (row[b] < rows);
                const int rr = valid[b] ? row[b] : 0;
                crow[b] = codes + (int64_t)rr * crb;
                srow[b] = scales + (int64_t)rr * srb;
            }
            float acc[R][MT];
            rows_dot<FMT, DEC, Q, MT, R, false>(crow, srow, U, lr, LPR, xr, xr, L, acc);
#pragma unroll
            for (int b = 0; b < R; ++b) {
                if (!valid[b] || lr != 0) continue;
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    if (t0 + t >= B) continue;
                    const int64_t o = (int64_t)(t0 + t) * rows + row[b];
                    if (out_f32) reinterpret_cast<float *>(y)[o] = acc[b][t];
                    else reinterpret_cast<uint16_t *>(y)[o] = f32_to_bf16_rne(acc[b][t]);
                }
            }
        }
    }
}

template <int FMT, int DEC, int Q, int MT>
static hipError_t gemv_go(const uint8_t *codes, const uint8_t *scales, int rows, int cols, const uint16_t *x, int B,
                          void *y, int out_f32, hipStream_t s) {
    constexpr int R = 2;
    const int U = cols / 32, LPR = lanes_per_row(U), RPW = WAVE / LPR;
    const int ngroups = (rows + RPW - 1) / RPW;
    int blocks = (ngroups + 4 * R - 1) / (4 * R);
    if (blocks > 256 * 16) blocks = 256 * 16;
    hipLaunchKernelGGL((gemv_kernel<FMT, DEC, Q, MT, R>), dim3(blocks), dim3(256), 0, s, codes, scales, rows, cols, x,
                       B, y, out_f32);
    return hipGetLastError();
}

template <int FMT, int DEC>
static hipError_t gemv_q(const uint8_t *codes, const uint8_t *scales, int rows, int cols, const uint16_t *x, int B,
                         void *y, int out_f32, hipStream_t s) {
    const int U = cols / 32, LPR = lanes_per_row(U), Q = (U + LPR - 1) / LPR;
    const bool one = (B == 1);
#define GO(QQ)                                                                                    \
    if (Q == QQ) {                                                                                \
        if (one) return gemv_go<FMT, DEC, QQ, 1>(codes, scales, rows, cols, x, B, y, out_f32, s); \
        return gemv_go<FMT, DEC, QQ, 4>(codes, scales, rows, cols, x, B, y, out_f32, s);          \
    }
    GO(1) GO(2) GO(3) GO(4)
#undef GO
    return hipErrorInvalidValue;
}

hipError_t launch_gemv(int fmt, int dec, const uint8_t *codes, const uint8_t *scales, int rows, int cols,
                       const uint16_t *x, int B, void *y, int out_f32, hipStream_t s) {
    if (fmt == FMT_E2M1) {
        if (dec == DEC_HW) return gemv_q<FMT_E2M1, DEC_HW>(codes, scales, rows, cols, x, B, y, out_f32, s);
        return gemv_q<FMT_E2M1, DEC_LUT>(codes, scales, rows, cols, x, B, y, out_f32, s);
    }
    if (dec == DEC_HW) return gemv_q<FMT_E2M3, DEC_HW>(codes, scales, rows, cols, x, B, y, out_f32, s);
    return gemv_q<FMT_E2M3, DEC_LUT>(codes, scales, rows, cols, x, B, y, out_f32, s);
}

}  // namespace moeq
