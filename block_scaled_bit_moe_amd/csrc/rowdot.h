// rowdot.h -- the streaming inner loop shared by the GEMV and the expert
// kernels: LPR lanes cooperate on one row, each taking the 32-weight units
// u = lr, lr + LPR, ... (up to Q of them); consecutive lanes read consecutive
// units, so a wave's loads of one row are contiguous.  Activations for the
// lane's units sit in registers for the whole pass (they are the same for
// every row).  R rows are loaded before any is decoded so that R * Q unit
// loads per lane are in flight.  The lane partial sums are combined by a
// DPP butterfly over the LPR lanes, identical for every row and every token;
// the sum is valid in the first lane of each row's lane group.
#pragma once

#include "common.h"

namespace moeq {

// Load the activation units (bf16, 64 bytes per unit) of MT tokens.
// rowptr[t] points at token t's row (nullptr: zeros).
template <int Q, int MT>
__device__ inline void load_x_units(u32 (&xr)[Q][MT][16], const uint16_t *const (&rowptr)[MT], int U, int lr,
                                    int LPR) {
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int u = lr + LPR * q;
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            if (u < U && rowptr[t]) {
                const uint4 *p = reinterpret_cast<const uint4 *>(rowptr[t] + 32 * (int64_t)u);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    uint4 a = p[v];
                    xr[q][t][4 * v + 0] = a.x;
                    xr[q][t][4 * v + 1] = a.y;
                    xr[q][t][4 * v + 2] = a.z;
                    xr[q][t][4 * v + 3] = a.w;
                }
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i) xr[q][t][i] = 0u;
            }
        }
    }
}

// acc[b][t] = row_b . x_t for R rows and MT tokens.  With SPLIT the activation
// is an fp32 vector carried as bf16 hi + lo parts (xh, xl) and both are used.
template <int FMT, int DEC, int Q, int MT, int R, bool SPLIT>
__device__ inline void rows_dot(const uint8_t *const (&crow)[R], const uint8_t *const (&srow)[R], int U, int lr,
                                int LPR, const u32 (&xh)[Q][MT][16], const u32 (&xl)[Q][MT][16], const Luts &L,
                                float (&acc)[R][MT]) {
    Unit<FMT> un[R][Q];
#pragma unroll
    for (int b = 0; b < R; ++b)
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int u = lr + LPR * q;
            if (u < U) load_unit<FMT>(un[b][q], crow[b], srow[b], u);
        }
#pragma unroll
    for (int b = 0; b < R; ++b)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[b][t] = 0.f;
#pragma unroll
    for (int b = 0; b < R; ++b) {
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int u = lr + LPR * q;
            if (u < U) {
                u32 w[16];
                decode_unit<FMT, DEC>(un[b][q], L, w);
                float s0, s1;
                unit_scales<FMT>(un[b][q], L, s0, s1);
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    if constexpr (SPLIT) acc[b][t] = unit_dot_split<FMT>(w, xh[q][t], xl[q][t], s0, s1, acc[b][t]);
                    else acc[b][t] = unit_dot<FMT>(w, xh[q][t], s0, s1, acc[b][t]);
                }
            }
        }
    }
#pragma unroll
    for (int b = 0; b < R; ++b)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[b][t] = group_sum_dpp(acc[b][t], LPR);
}

// Lanes per row for a row of U units: the largest power of two <= min(64, U).
__host__ __device__ inline int lanes_per_row(int U) {
    int l = 64;
    while (l > U && l > 1) l >>= 1;
    return l;
}

}  // namespace moeq
