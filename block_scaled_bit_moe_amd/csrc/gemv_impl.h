// gemv_impl.h -- dense_gemv_q: y[b] = W x[b] for a block-scaled W and B <= 8 bf16
// tokens that share every decoded weight (knivesysl README, "formats": the fp6
// e2m3 projections with a power-of-two scale per 128; Strata docs/INTEL.md,
// "Decode round 2": aligned 16-byte weight loads, codebook lookups kept off the
// critical path).
//
// Bandwidth-bound: every weight byte is read from HBM once per pass of up to
// eight tokens.  One token: x stays in registers and each wave streams its
// row groups (register pipeline, two workgroups per CU).  Several tokens: their
// x does not fit in registers, so one 16-wave workgroup per CU holds it in LDS
// and deals its row range to the waves (measured on the 25600 x 5120 e2m3
// matrix: B=4 in 35 us against 59 us for a 4-wave LDS-ring design; B=1 in 23
// us with the register pipeline against 24 us with the 16-wave kernel).
#pragma once

#include "kernels.h"
#include "rowdot.h"

#include <algorithm>
#include <type_traits>

namespace moeq {

constexpr int GEMV_REG_WG_PER_CU = 2;   // one-token kernel: workgroups per CU (its occupancy)

static int num_cus() { return cached_cus(); }

// Register-streamed variant: the x units stay in VGPRs, and each wave walks
// its rows (every nw-th row group) R per pass with the next pass's loads in
// flight (RowPipe).  A grid of a few workgroups per CU, so every wave streams
// many rows after loading x once.  Used for one token.
template <int FMT, int DEC, int Q, int MT, int R>
__global__ __launch_bounds__(256) void gemv_reg_kernel(const uint8_t *__restrict__ codes,
                                                   const uint8_t *__restrict__ scales, int rows, int cols,
                                                   const uint16_t *__restrict__ x, int B, void *__restrict__ y,
                                                   int out_f32) {
    constexpr int PAIR = (DEC == DEC_LUT) ? (Fmt<FMT>::SIX ? LUT_E2M3_PAIR : LUT_E2M1_PAIR) : 1;
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
    if (gw >= ngroups) return;   // uniform over the wave; no barrier follows
    const int npass = (ngroups - gw + nw * R - 1) / (nw * R);

    for (int t0 = 0; t0 < B; t0 += MT) {
        u32 xr[Q][MT][16];
        const uint16_t *xp[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) xp[t] = (t0 + t < B) ? x + (int64_t)(t0 + t) * cols : nullptr;
        load_x_units<Q, MT>(xr, xp, U, lr, LPR);

        // pass p, slot b: row group gw + (p * R + b) * nw (past the end: row 0, result dropped)
        auto row = [&](int p, int b, const uint8_t *&c, const uint8_t *&sc) -> int {
            const int grp = gw + (p * R + b) * nw;
            const int r = grp * RPW + rsub;
            const bool ok = grp < ngroups && r < rows;
            const int rr = ok ? r : 0;
            c = codes + (int64_t)rr * crb;
            sc = scales + (int64_t)rr * srb;
            return ok ? r : -1;
        };
        auto out = [&](int, int, int r, const float (&acc)[MT]) {
            if (r < 0 || lr != 0) return;
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                if (t0 + t >= B) continue;
                const int64_t o = (int64_t)(t0 + t) * rows + r;
                if (out_f32) reinterpret_cast<float *>(y)[o] = acc[t];
                else reinterpret_cast<uint16_t *>(y)[o] = f32_to_bf16_rne(acc[t]);
            }
        };
        RowPipe<FMT, DEC, Q, MT, R, false> pipe;
        pipe.begin(row, U, lr, LPR);
        pipe.run(npass, row, U, lr, LPR, xr, xr, L, out);
    }
}

template <int FMT, int DEC, int Q, int MT>
static hipError_t gemv_reg_go(const uint8_t *codes, const uint8_t *scales, int rows, int cols, const uint16_t *x, int B,
                          void *y, int out_f32, hipStream_t s) {
    constexpr int R = 2;
    const int U = cols / 32, LPR = lanes_per_row(U), RPW = WAVE / LPR;
    const int ngroups = (rows + RPW - 1) / RPW;
    // enough waves to fill the CUs, each with several passes to stream
    int blocks = (ngroups + 4 * R - 1) / (4 * R);
    const int cap = num_cus() * GEMV_REG_WG_PER_CU;
    if (blocks > cap) blocks = cap;
    hipLaunchKernelGGL((gemv_reg_kernel<FMT, DEC, Q, MT, R>), dim3(blocks), dim3(256), 0, s, codes, scales, rows, cols, x,
                       B, y, out_f32);
    return hipGetLastError();
}

// 16-wave variant: one workgroup per CU streams a contiguous range of rows;
// the tokens of a pass sit in LDS, unit-major (unit u of token t at word
// u * (16 * xt + 4) + 16 t: the 4-word pad puts 16 consecutive units on 16
// different bank groups, and a lane reads every token of its unit at
// immediate offsets from one address).  Rows are dealt to the waves R at a
// time from an LDS counter, with two items in flight per wave, so waves whose
// loads are served sooner take more rows and all finish together.  The
// arithmetic of a row is the register-streamed kernel's (same lanes, units,
// order and reduction), so every token's result is the same for any batch.
constexpr int GL_XT = 8;
constexpr size_t GL_LDS = 100 * 1024;
// Waves per workgroup and rows per item (each x unit read from LDS once for
// all rows of an item).  Measured at B = 4 on the 25600 x 5120 e2m3 matrix:
// 16 waves, 1 row 34.6 us; 16 waves, 2 rows 57.8; 8 waves, 2 rows 38.6;
// 8 waves, 4 rows 58.9 (more rows per item cost registers, not LDS time).
constexpr int GL_NW = 16;
constexpr int GL_RX = 1;

template <int FMT, int DEC, int Q, int R, int NW>
__global__ __launch_bounds__(64 * NW) void gemv_lds_kernel(const uint8_t *__restrict__ codes,
                                                        const uint8_t *__restrict__ scales, int rows, int cols,
                                                        const uint16_t *__restrict__ x, int B, void *__restrict__ y,
                                                        int out_f32, int xt) {
    constexpr int PAIR = (DEC == DEC_LUT) ? (Fmt<FMT>::SIX ? LUT_E2M3_PAIR : LUT_E2M1_PAIR) : 1;
    __shared__ u32 s_pair[PAIR];
    __shared__ float s_scale[LUT_SCALE];
    __shared__ int s_next[2];
    extern __shared__ __attribute__((aligned(16))) u32 s_x[];
    const Luts L{s_pair, s_scale};
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (tid == 0) {
        s_next[0] = 0;
        s_next[1] = 0;
    }
    build_luts<FMT>(L, tid, 64 * NW, DEC == DEC_LUT);

    const int U = cols / 32, LPR = lanes_per_row(U), RPW = WAVE / LPR;
    const int lr = lane & (LPR - 1), rs = lane / LPR;
    const int64_t crb = Fmt<FMT>::code_row_bytes(cols), srb = Fmt<FMT>::scale_row_bytes(cols);
    const int US = 16 * xt + 4;
    const int r0 = (int)((int64_t)rows * blockIdx.x / gridDim.x);
    const int nrow = (int)((int64_t)rows * (blockIdx.x + 1) / gridDim.x) - r0;
    const int nitem = (nrow + R * RPW - 1) / (R * RPW);
    // row b of item it for this lane group (past the range: the first row, result dropped)
    auto jrow = [&](int it, int b) { return (it * R + b) * RPW + rs; };

    int nb = 0;
    for (int t0 = 0; t0 < B; t0 += xt) {
        const int mb = min(xt, B - t0);
        auto grab = [&]() -> int {
            int v = 0;
            if (lane == 0) v = atomicAdd(&s_next[nb & 1], 1);
            return __builtin_amdgcn_readfirstlane(v);
        };
        Unit<FMT> un[2][R][Q];
        auto issue = [&](int st, int it) {
#pragma unroll
            for (int b = 0; b < R; ++b) {
                const int j = jrow(it, b);
                const int64_t r = r0 + (j < nrow ? j : 0);
                const uint8_t *c = codes + r * crb, *sc = scales + r * srb;
#pragma unroll
                for (int q = 0; q < Q; ++q) {
                    const int u = lr + LPR * q;
                    load_unit<FMT>(un[st][b][q], c, sc, u < U ? u : lr);
                }
            }
        };
        auto compute = [&](int st, int it) {
            float acc[R][GL_XT];
#pragma unroll
            for (int b = 0; b < R; ++b)
#pragma unroll
                for (int t = 0; t < GL_XT; ++t) acc[b][t] = 0.f;
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const int u = lr + LPR * q;
                // this lane's unit of each row, decoded once; each x unit read once for all rows
                u32 wd[R][16];
                float s0[R], s1[R];
#pragma unroll
                for (int b = 0; b < R; ++b) {
                    decode_unit<FMT, DEC>(un[st][b][q], L, wd[b]);
                    unit_scales<FMT>(un[st][b][q], L, s0[b], s1[b]);
                }
                const uint4 *xb = reinterpret_cast<const uint4 *>(s_x + (u < U ? u : 0) * US);
#pragma unroll
                for (int t = 0; t < GL_XT; ++t) {
                    if (t < mb) {
                        u32 xv[16];
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const uint4 A = xb[4 * t + v];
                            xv[4 * v] = A.x; xv[4 * v + 1] = A.y; xv[4 * v + 2] = A.z; xv[4 * v + 3] = A.w;
                        }
#pragma unroll
                        for (int b = 0; b < R; ++b) {
                            const float d = unit_dot<FMT>(wd[b], xv, s0[b], s1[b], acc[b][t]);
                            acc[b][t] = u < U ? d : acc[b][t];
                        }
                    }
                }
            }
#pragma unroll
            for (int b = 0; b < R; ++b) {
                const int j = jrow(it, b);
#pragma unroll
                for (int t = 0; t < GL_XT; ++t) {
                    if (t < mb) {
                        const float v = group_sum_dpp(acc[b][t], LPR);
                        if (j < nrow && lr == 0) {
                            const int64_t o = (int64_t)(t0 + t) * rows + r0 + j;
                            if (out_f32) reinterpret_cast<float *>(y)[o] = v;
                            else reinterpret_cast<uint16_t *>(y)[o] = f32_to_bf16_rne(v);
                        }
                    }
                }
            }
        };
        // Pass over tokens t0 .. t0+mb-1.  Its counter was cleared at the start of the
        // previous pass (or kernel); the other one is cleared now, after the barrier
        // that every wave passes only once done with it.
        __syncthreads();
        if (tid == 0) s_next[(nb + 1) & 1] = 0;
        int ia = grab();
        issue(0, ia);   // the weights do not depend on x: in flight while x is staged
        for (int q = tid; q < mb * U * 4; q += 64 * NW) {
            const int t = q / (U * 4), rem = q - t * (U * 4), u = rem >> 2, v = rem & 3;
            const uint4 val = *reinterpret_cast<const uint4 *>(x + (int64_t)(t0 + t) * cols + 32 * u + 8 * v);
            *reinterpret_cast<uint4 *>(s_x + u * US + 16 * t + 4 * v) = val;
        }
        __syncthreads();
        for (;;) {
            const int ib = grab();
            issue(1, ib);
            if (ia >= nitem) break;
            compute(0, ia);
            ia = grab();
            issue(0, ia);
            if (ib >= nitem) break;
            compute(1, ib);
        }
        ++nb;
    }
}

template <int FMT, int DEC, int Q>
static hipError_t gemv_lds_go(const uint8_t *codes, const uint8_t *scales, int rows, int cols, const uint16_t *x, int B,
                              void *y, int out_f32, hipStream_t s) {
    constexpr int R = (Q >= 2) ? GL_RX : 2 * GL_RX;
    auto kern = gemv_lds_kernel<FMT, DEC, Q, R, GL_NW>;
    const int U = cols / 32;
    int xt = std::min(B, GL_XT);
    while (xt > 1 && (size_t)U * (16 * xt + 4) * 4 > GL_LDS) --xt;
    const size_t dyn = (size_t)U * (16 * xt + 4) * 4;
    // dynamic LDS beyond the default limit (raised once per device)
    const hipError_t le = ensure_dyn_lds(reinterpret_cast<const void *>(kern), dyn);
    if (le != hipSuccess) return le;
    const int RPW = WAVE / lanes_per_row(U);
    // one workgroup per CU, at least a few rows per wave
    const int G = std::max(1, std::min(num_cus(), rows / (4 * GL_NW * RPW)));
    hipLaunchKernelGGL(kern, dim3(G), dim3(64 * GL_NW), dyn, s, codes, scales, rows, cols, x, B, y, out_f32, xt);
    return hipGetLastError();
}

template <int FMT, int DEC>
hipError_t gemv_q(const uint8_t *codes, const uint8_t *scales, int rows, int cols, const uint16_t *x, int B,
                         void *y, int out_f32, hipStream_t s) {
    const int U = cols / 32, LPR = lanes_per_row(U), Q = (U + LPR - 1) / LPR;
    const bool one = (B == 1);
#define GO(QQ)                                                                                    \
    if (Q == QQ) {                                                                                \
        if (one) return gemv_reg_go<FMT, DEC, QQ, 1>(codes, scales, rows, cols, x, B, y, out_f32, s); \
        return gemv_lds_go<FMT, DEC, QQ>(codes, scales, rows, cols, x, B, y, out_f32, s);             \
    }
    GO(1) GO(2) GO(3) GO(4)
#undef GO
    return hipErrorInvalidValue;
}

}  // namespace moeq

#define MOEQ_GEMV_INSTANCE(F)                                                                                  \
    namespace moeq {                                                                                           \
    template <> GemvFn gemv_fn_for<F, DEC_HW>() { return gemv_q<F, DEC_HW>; }                                  \
    template <> GemvFn gemv_fn_for<F, DEC_LUT>() { return gemv_q<F, DEC_LUT>; }                                \
    }
