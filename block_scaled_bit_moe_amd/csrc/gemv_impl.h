// gemv_impl.h -- dense_gemv_q: y[b] = W x[b] for a block-scaled W and B <= 8 bf16
// tokens that share every decoded weight (knivesysl README, "formats": the fp6
// e2m3 projections with a power-of-two scale per 128; Strata docs/INTEL.md,
// "Decode round 2": aligned 16-byte weight loads, codebook lookups kept off the
// critical path).
//
// Bandwidth-bound: every weight byte is read from HBM once per pass of up to
// eight tokens.  One token: x stays in registers and each wave streams its
// row groups (register pipeline, two workgroups per CU).  Several tokens with
// the hardware conversions: the matrix-core kernel (gemv_mfma_kernel), which
// decodes a unit once for all tokens.  Several tokens with the LDS tables (or
// rows of an odd number of units): one 16-wave workgroup per CU holds x in LDS
// and deals its row range to the waves with the one-token kernel's dot2
// arithmetic (measured on the 25600 x 5120 e2m3 matrix: B=4 in 35 us against
// 59 us for a 4-wave LDS-ring design; B=1 in 23 us with the register pipeline
// against 24 us with the 16-wave kernel).  The matrix cores add a row's
// products in another order than the dot2 kernels, so with the hardware
// conversions a token's result at B > 1 can differ in the last bits from the
// same token alone (both are within the format's error bound of the exact
// value); with the LDS tables every token's result is the same for any batch.
#pragma once

#include "kernels.h"
#include "memops.h"
#include "mfma_unit.h"
#include "rowdot.h"

#include <algorithm>
#include <type_traits>
#include <utility>

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
    // one row per lane group and pass (the next pass's row in flight meanwhile):
    // on the 25600 x 5120 e2m3 matrix 19.6 us, against 21.3 with two rows per
    // pass and 24-34 us with three or four rows or more workgroups per CU
    // (the more rows a CU has open at once, the slower)
    constexpr int R = 1;
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

// Matrix-core variant for two or more tokens (hardware conversions): the
// tokens of a pass are the rows of the A operand of v_mfma_f32_16x16x32_bf16
// and 16 weight rows its B operand, so a weight unit is decoded once and meets
// all tokens in four instructions instead of 16 dot2 per token.
//
// The eight waves of a workgroup share one 16-row tile at a time and split its
// K steps round robin (wave w takes steps w, w + 8, ...), so a workgroup reads
// each of its 16 rows front to back as one stream: at most 16 rows per CU are
// being read at any time.  Measured at B = 4 on the 25600 x 5120 e2m3 matrix:
// a tile per wave (128 rows open per CU) took 29.5-46 us, slower the more
// loads were in flight; the shared tile takes 25.8 us with 1-2 steps per wave
// in flight and 29.6 us with 5 (the dot2 kernel below: 32.0 us).  The same
// with four units per lane (384-byte runs per row) took 31.1 us, and four or
// sixteen waves per workgroup 28.8 and 79 us.  A step is 4 * UPL units of the
// tile's rows: lane (g, n) loads the UPL consecutive units UPL * (4s + g) ..
// + UPL - 1 of row n (four lane groups: one run of 4 * UPL units per row),
// converts them with the block scale folded in exactly (pf_unit_to_b), and
// MFMA (t, q) of the step takes weights 8q .. 8q+7 of unit UPL * (4s + g) + t
// in lane group g.  Lane (g, m) reads the same K range of token m from LDS
// (unit-major, as the 16-wave kernel stages it).  Units past the row's end are
// zero on both sides.  Each wave's sums of a tile go to LDS when its last step
// of the tile is done; after the workgroup's tiles (GM_MT at a time) the eight
// partial sums of every output are added in wave order, so the result does not
// depend on timing.  The loads run NST - 1 of the wave's steps ahead in a ring
// of register stages, across tile boundaries.
constexpr int GM_NW = 8;                 // waves per workgroup, one workgroup per CU
constexpr int GM_MT = 8;                 // tiles whose partial sums a workgroup holds in LDS at once
constexpr int GM_XB = 4;                 // token pieces per thread loaded at once when staging
constexpr size_t GM_PART = (size_t)GM_MT * GM_NW * 256 * 4;    // bytes of partial sums
constexpr size_t GM_LDS = 150 * 1024 - GM_PART;                // staged tokens of a pass
template <int FMT> constexpr int gm_upl() { return 2; }
// ring of three stages (two steps ahead) for every code width: four-bit codes
// 22.0 us at B = 4 against 23.2 with four stages and 24.7 with six (e2m1)
template <int FMT> constexpr int gm_nst() { return 3; }

// Units u0 .. u0 + UPL - 1 (u0 a multiple of UPL) of a row: one contiguous run
// of code bytes, and in sw the two aligned scale words that hold the scale
// bytes of all of them (read through a buffer resource, so they may reach past
// the array's end).  The bytes are picked out by unit_run_scales where the
// units are used: until then the loaded registers see no operation (not even
// the zero extension of a byte load), so the compiler has nothing to place
// ahead of their use, where it would wait for every younger load.  Returns the
// bit offset of the first scale byte in the two words.
template <int FMT, int UPL>
__device__ inline u32 load_unit_run(Unit<FMT> (&w)[UPL], u32 (&sw)[2], const uint8_t *codes,
                                    __amdgpu_buffer_rsrc_t srs, u32 srow, int u0) {
    using F = Fmt<FMT>;
    if constexpr (!F::SIX) {
        const uint4 *p = reinterpret_cast<const uint4 *>(codes + (int64_t)u0 * 16);
#pragma unroll
        for (int t = 0; t < UPL; ++t) w[t].c = p[t];
    } else {
        static_assert(UPL % 2 == 0, "six-bit units are loaded in 48-byte pairs");
        const uint4 *p = reinterpret_cast<const uint4 *>(codes + (int64_t)u0 * 24);
#pragma unroll
        for (int t = 0; t < UPL; t += 2) {
            const uint4 q0 = p[3 * (t / 2)], q1 = p[3 * (t / 2) + 1], q2 = p[3 * (t / 2) + 2];
            w[t].c0 = make_uint2(q0.x, q0.y);
            w[t].c1 = make_uint2(q0.z, q0.w);
            w[t].c2 = make_uint2(q1.x, q1.y);
            w[t + 1].c0 = make_uint2(q1.z, q1.w);
            w[t + 1].c1 = make_uint2(q2.x, q2.y);
            w[t + 1].c2 = make_uint2(q2.z, q2.w);
        }
    }
    u32 off;
    if constexpr (F::TWO_SCALES) off = 2u * (u32)u0;                        // two bytes per unit
    else if constexpr (F::SCALE == SC_FP16) off = 2u * (u32)(u0 >> 1);     // an fp16 per two units
    else off = (u32)(u0 / (F::BLOCK / 32));                                  // a byte per BLOCK / 32 units
    off += srow;
    sw[0] = __builtin_amdgcn_raw_buffer_load_b32(srs, (int)(off & ~3u), 0, 0);
    if constexpr (F::TWO_SCALES || (UPL > 2 && (F::SCALE == SC_FP16 || F::BLOCK == 32)))
        sw[1] = __builtin_amdgcn_raw_buffer_load_b32(srs, (int)((off & ~3u) + 4u), 0, 0);
    else
        sw[1] = 0u;
    return (off & 3u) * 8u;
}

// The scale bits of each unit of a run, from its two scale words.
template <int FMT, int UPL>
__device__ inline void unit_run_scales(Unit<FMT> (&w)[UPL], const u32 (&sw)[2], u32 sh) {
    using F = Fmt<FMT>;
    const uint64_t v = (((uint64_t)sw[1] << 32) | sw[0]) >> sh;
#pragma unroll
    for (int t = 0; t < UPL; ++t) {
        if constexpr (F::TWO_SCALES) w[t].s = (u32)(v >> (16 * t)) & 0xFFFFu;
        else if constexpr (F::SCALE == SC_FP16) w[t].s = (u32)(v >> (16 * (t / 2))) & 0xFFFFu;
        else if constexpr (F::BLOCK == 32) w[t].s = (u32)(v >> (8 * t)) & 0xFFu;
        else w[t].s = (u32)v & 0xFFu;    // one block holds the whole run (BLOCK / 32 a multiple of UPL)
    }
}

template <int FMT, int NST, int UPL>
__global__ __launch_bounds__(64 * GM_NW, 1) void gemv_mfma_kernel(const uint8_t *__restrict__ codes,
                                                               const uint8_t *__restrict__ scales, int rows, int cols,
                                                               const uint16_t *__restrict__ x, int B,
                                                               void *__restrict__ y, int out_f32, int xt) {
    __shared__ float s_scale[LUT_SCALE];
    extern __shared__ __attribute__((aligned(16))) u32 s_x[];
    constexpr bool WLO = pf_split_w<FMT>();
    constexpr int KU = 4 * UPL;                    // units per K step
    static_assert(Fmt<FMT>::BLOCK < 128 || (Fmt<FMT>::BLOCK / 32) % UPL == 0, "a run inside one scale block");
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    if constexpr (Fmt<FMT>::SCALE == SC_E4M3) {   // the other scales are converted arithmetically
        Luts Lt;
        Lt.pair = nullptr;
        Lt.scale = s_scale;
        build_luts<FMT>(Lt, tid, 64 * GM_NW, false);
    }
    const int U = cols / 32, S = (U + KU - 1) / KU;   // units per row (a multiple of UPL), K steps
    const int US = 16 * xt + 4;                    // words per staged unit: xt tokens and a pad
    float *s_part = reinterpret_cast<float *>(s_x + (size_t)U * US);   // [GM_MT][GM_NW][64 lanes][4]
    const int64_t crb = Fmt<FMT>::code_row_bytes(cols), srb = Fmt<FMT>::scale_row_bytes(cols);
    const int ntile = (rows + 15) >> 4;
    const int tb = (int)((int64_t)ntile * blockIdx.x / gridDim.x);
    const int te = (int)((int64_t)ntile * (blockIdx.x + 1) / gridDim.x);
    const int nw_used = min(GM_NW, S);             // waves that own steps of a tile
    const int per_tile = wv < S ? (S - wv + GM_NW - 1) / GM_NW : 0;   // this wave's steps of each tile
    const int g = lane >> 4, n = lane & 15;        // lane group (K); row of the tile (B) and token (A)
    const __amdgpu_buffer_rsrc_t srs = rsrc_of(scales, (uint64_t)rows * srb);

    for (int t0 = 0; t0 < B; t0 += xt) {
        const int mb = min(xt, B - t0);
        bool staged = false;
        for (int j0 = tb; j0 < te; j0 += GM_MT) {
            const int nt = min(GM_MT, te - j0);
            const int nstep = nt * per_tile;           // (tile, K step) pairs of this wave in this group
            Unit<FMT> wq[NST][UPL];
            u32 wsw[NST][2], wsh[NST];
            int i_tile = j0, i_s = wv;                 // next (tile, step) to load; past the end the last one again
            auto issue = [&](auto sc) {
                constexpr int K = decltype(sc)::value;
                const int row = min(i_tile * 16 + n, rows - 1);
                const int u0 = min(KU * i_s + UPL * g, U - UPL);
                wsh[K] = load_unit_run<FMT, UPL>(wq[K], wsw[K], codes + (int64_t)row * crb, srs, (u32)(row * srb), u0);
                i_s += GM_NW;
                if (i_s >= S) {
                    i_s = wv;
                    i_tile = min(i_tile + 1, j0 + nt - 1);
                }
            };
            __syncthreads();   // the previous group is done with s_part (and the scale table is built)
            // The first NST - 1 steps' weight loads go out before the tokens are
            // staged (they do not depend on them), in step order, so that stage 0's
            // loads are the oldest in flight as on every later pass of the ring.
            if (nstep > 0)
                [&]<int... I>(std::integer_sequence<int, I...>) {
                    ((__builtin_amdgcn_sched_barrier(0), issue(std::integral_constant<int, I>{})), ...);
                }(std::make_integer_sequence<int, NST - 1>{});
            __builtin_amdgcn_sched_barrier(0);
            if (!staged) {
                // The pass's tokens into LDS: GM_XB loads per thread in flight at
                // once, then their stores (past the end: the last piece again, not stored).
                const int npc = mb * U * 4;
                for (int q0 = tid; q0 < npc; q0 += 64 * GM_NW * GM_XB) {
                    uint4 v[GM_XB];
#pragma unroll
                    for (int j = 0; j < GM_XB; ++j) {
                        const int q = min(q0 + j * 64 * GM_NW, npc - 1);
                        const int t = q / (U * 4), rem = q - t * (U * 4), uu = rem >> 2, vv = rem & 3;
                        v[j] = *reinterpret_cast<const uint4 *>(x + (int64_t)(t0 + t) * cols + 32 * uu + 8 * vv);
                    }
#pragma unroll
                    for (int j = 0; j < GM_XB; ++j) {
                        const int q = q0 + j * 64 * GM_NW;
                        if (q < npc) {
                            const int t = q / (U * 4), rem = q - t * (U * 4), uu = rem >> 2, vv = rem & 3;
                            *reinterpret_cast<uint4 *>(s_x + uu * US + 16 * t + 4 * vv) = v[j];
                        }
                    }
                }
                __syncthreads();
                staged = true;
            }
            const int tm = min(n, mb - 1);         // A rows past the pass's tokens repeat one; their sums are dropped

            f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
            int c_j = 0, c_k = 0, c_s = wv;         // tile (in the group), its step count so far, K step
            // One (tile, step): start the load NST - 1 steps ahead into the stage the
            // previous step freed, then multiply this step's units.  The loads are
            // unconditional (past the end they repeat the last step's addresses)
            // and only the arithmetic depends on `live`, so every pass of the loop
            // below takes one path through the ring and the compiler keeps each
            // stage in the same registers (and counts exactly which loads are still
            // in flight).  No instruction crosses a step boundary: a load moved
            // above the previous step's use of the same stage would need other
            // registers, and copies of the whole ring on every pass of the loop.
            auto step = [&](auto sc, bool live) {
                constexpr int K = decltype(sc)::value;
                __builtin_amdgcn_sched_barrier(0);
                issue(std::integral_constant<int, (K + NST - 1) % NST>{});
                if (!live) return;
                unit_run_scales<FMT, UPL>(wq[K], wsw[K], wsh[K]);
#pragma unroll
                for (int t = 0; t < UPL; ++t) {
                    const int u = KU * c_s + UPL * g + t;
                    const bool ok = u < U;
                    Unit<FMT> w = wq[K][t];
                    if (!ok) pf_zero_unit<FMT>(w);
                    bf16x8_t bw[4], bwl[4];
                    pf_unit_to_b<FMT>(w, s_scale, bw, bwl);
                    const uint4 *xa = reinterpret_cast<const uint4 *>(s_x + (ok ? u : 0) * US + 16 * tm);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        uint4 av = xa[q];
                        if (!ok) av = make_uint4(0u, 0u, 0u, 0u);
                        const bf16x8_t A = __builtin_bit_cast(bf16x8_t, av);
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, bw[q], acc, 0, 0, 0);
                        if (WLO) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, bwl[q], acc, 0, 0, 0);
                    }
                }
                c_s += GM_NW;
                if (++c_k == per_tile) {
                    // this wave's sums of the tile: lane (g, n) holds tokens 4g .. 4g+3 of row n
                    *reinterpret_cast<f32x4_t *>(s_part + ((size_t)(c_j * GM_NW + wv) * 64 + lane) * 4) = acc;
                    acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
                    c_k = 0;
                    c_s = wv;
                    ++c_j;
                }
            };
            for (int f = 0; f < nstep; f += NST)
                [&]<int... I>(std::integer_sequence<int, I...>) {
                    (step(std::integral_constant<int, I>{}, f + I < nstep), ...);
                }(std::make_integer_sequence<int, NST>{});
            __syncthreads();
            // every output of the group's tiles: the waves' partial sums in wave order
            for (int e = tid; e < nt * 256; e += 64 * GM_NW) {
                const int jj = e >> 8, r = (e >> 4) & 15, m = e & 15;
                const int row = (j0 + jj) * 16 + r;
                if (m >= mb || row >= rows) continue;
                const int pl = 16 * (m >> 2) + r, pi = m & 3;     // lane and element of (token m, row r)
                float v = 0.f;
                for (int w = 0; w < nw_used; ++w) v += s_part[((size_t)(jj * GM_NW + w) * 64 + pl) * 4 + pi];
                const int64_t o = (int64_t)(t0 + m) * rows + row;
                if (out_f32) reinterpret_cast<float *>(y)[o] = v;
                else reinterpret_cast<uint16_t *>(y)[o] = f32_to_bf16_rne(v);
            }
        }
    }
}

template <int FMT>
static hipError_t gemv_mfma_go(const uint8_t *codes, const uint8_t *scales, int rows, int cols, const uint16_t *x,
                               int B, void *y, int out_f32, hipStream_t s) {
    auto kern = gemv_mfma_kernel<FMT, gm_nst<FMT>(), gm_upl<FMT>()>;
    const int U = cols / 32;
    int xt = std::min(B, GL_XT);
    while (xt > 1 && (size_t)U * (16 * xt + 4) * 4 > GM_LDS) --xt;
    const size_t dyn = (size_t)U * (16 * xt + 4) * 4 + GM_PART;
    const hipError_t le = ensure_dyn_lds(reinterpret_cast<const void *>(kern), dyn);
    if (le != hipSuccess) return le;
    const int ntile = (rows + 15) / 16;
    // the fewest workgroups (at most one per CU) that give none more tiles
    // than one per CU would: 25600 rows, 1600 tiles, 229 workgroups of 7
    // instead of 256 of 6 or 7 (25.55 against 25.88 us; 200 of 8: 27.3 us)
    int G = std::max(1, std::min(num_cus(), ntile));
    const int per = (ntile + G - 1) / G;
    G = (ntile + per - 1) / per;
    hipLaunchKernelGGL(kern, dim3(G), dim3(64 * GM_NW), dyn, s, codes, scales, rows, cols, x, B, y, out_f32, xt);
    return hipGetLastError();
}

template <int FMT, int DEC>
hipError_t gemv_q(const uint8_t *codes, const uint8_t *scales, int rows, int cols, const uint16_t *x, int B,
                         void *y, int out_f32, hipStream_t s) {
    const int U = cols / 32, LPR = lanes_per_row(U), Q = (U + LPR - 1) / LPR;
    const bool one = (B == 1);
    // The matrix-core kernel loads runs of gm_upl units: rows must hold a whole
    // number of them.  int4 + fp16 weights enter it as two bf16 parts (twice
    // the instructions, and an fp32 product per weight to split), which only
    // pays above four tokens (25600 x 5120: B = 2, 4, 8 in 39.3, 40.3, 42.0 us
    // against 28.5, 37.6, 56.3 us with the dot2 kernel).
    if constexpr (DEC == DEC_HW)
        if (!one && U % gm_upl<FMT>() == 0 && (FMT != FMT_INT4 || B > 4))
            return gemv_mfma_go<FMT>(codes, scales, rows, cols, x, B, y, out_f32, s);
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
