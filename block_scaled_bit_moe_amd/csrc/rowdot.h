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

// Double-buffered row stream: passes of R rows per lane group, the loads of
// pass p+1 in flight while pass p is decoded and multiplied.  `row(p, b,
// &crow, &srow)` gives row b of pass p and returns its id, or -1 for a row
// past the end (then it must still point at a valid row: every load is
// issued, so the compiler can count the outstanding loads exactly and wait
// only for the pass it needs).  `out(p, b, id, acc)` receives the reduced
// sums (valid in the first lane of each lane group).  begin() issues pass 0
// early, e.g. before a wait that the weights do not depend on.
template <int FMT, int DEC, int Q, int MT, int R, bool SPLIT>
struct RowPipe {
    Unit<FMT> un[2][R][Q];
    int id[2][R];

    template <typename RowFn>
    __device__ inline void issue(int slot, int p, RowFn &row, int U, int lr, int LPR) {
#pragma unroll
        for (int b = 0; b < R; ++b) {
            const uint8_t *c, *sc;
            id[slot][b] = row(p, b, c, sc);
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const int u = lr + LPR * q;
                load_unit<FMT>(un[slot][b][q], c, sc, u < U ? u : 0);
            }
        }
    }

    template <typename OutFn>
    __device__ inline void compute(int slot, int p, int U, int lr, int LPR, const u32 (&xh)[Q][MT][16],
                                   const u32 (&xl)[Q][MT][16], const Luts &L, OutFn &out) {
        float acc[R][MT];
#pragma unroll
        for (int b = 0; b < R; ++b)
#pragma unroll
            for (int t = 0; t < MT; ++t) acc[b][t] = 0.f;
#pragma unroll
        for (int b = 0; b < R; ++b)
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const int u = lr + LPR * q;
                if (u < U) {
                    u32 w[16];
                    decode_unit<FMT, DEC>(un[slot][b][q], L, w);
                    float s0, s1;
                    unit_scales<FMT>(un[slot][b][q], L, s0, s1);
#pragma unroll
                    for (int t = 0; t < MT; ++t) {
                        if constexpr (SPLIT) acc[b][t] = unit_dot_split<FMT>(w, xh[q][t], xl[q][t], s0, s1, acc[b][t]);
                        else acc[b][t] = unit_dot<FMT>(w, xh[q][t], s0, s1, acc[b][t]);
                    }
                }
            }
#pragma unroll
        for (int b = 0; b < R; ++b) {
#pragma unroll
            for (int t = 0; t < MT; ++t) acc[b][t] = group_sum_dpp(acc[b][t], LPR);
            out(p, b, id[slot][b], acc[b]);
        }
    }

    template <typename RowFn>
    __device__ inline void begin(RowFn &row, int U, int lr, int LPR) { issue(0, 0, row, U, lr, LPR); }

    // passes 0 .. npass-1 (pass 0 already issued by begin)
    template <typename RowFn, typename OutFn>
    __device__ inline void run(int npass, RowFn &row, int U, int lr, int LPR, const u32 (&xh)[Q][MT][16],
                               const u32 (&xl)[Q][MT][16], const Luts &L, OutFn &out) {
        for (int p = 0; p < npass; p += 2) {
            issue(1, p + 1, row, U, lr, LPR);
            compute(0, p, U, lr, LPR, xh, xl, L, out);
            issue(0, p + 2, row, U, lr, LPR);
            compute(1, p + 1, U, lr, LPR, xh, xl, L, out);
        }
    }
};

// Lanes per row for a row of U units: the largest power of two <= min(64, U).
__host__ __device__ inline int lanes_per_row(int U) {
    int l = 64;
    while (l > U && l > 1) l >>= 1;
    return l;
}

}  // namespace moeq
