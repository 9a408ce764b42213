// gemv.hip -- dense_gemv_q: y[b] = W x[b] for a block-scaled W and B <= 8 bf16
// tokens that share every decoded weight (knivesysl README, "formats": the fp6
// e2m3 projections with a power-of-two scale per 128; Strata docs/INTEL.md,
// "Decode round 2": aligned 16-byte weight loads, codebook lookups kept off the
// critical path).
//
// Bandwidth-bound: every weight byte is read from HBM once per pass of MT
// tokens.  For several tokens each workgroup streams a contiguous range of row
// chunks through an LDS ring (stream.h): the x registers of 4 tokens leave no
// room for deep register pipelines.  One workgroup per CU (the ring takes most
// of the LDS), chunks split evenly over the workgroups.  For one token the
// register-pipelined kernel below is faster (measured: 25.5 vs 39.6 us on the
// 25600 x 5120 e2m3 matrix).
#include "kernels.h"
#include "rowdot.h"
#include "stream.h"

#include <type_traits>

namespace moeq {

constexpr int GEMV_L = 7;    // 16-byte loads per thread per chunk: 28 KiB stages
constexpr int GEMV_NS = 4;   // stages in flight
constexpr int GEMV_REG_WG_PER_CU = 2;   // one-token kernel: workgroups per CU (its occupancy)

template <int FMT, int DEC, int Q, int MT>
__global__ __launch_bounds__(256) void gemv_ring_kernel(const uint8_t *__restrict__ codes,
                                                   const uint8_t *__restrict__ scales, int rows, int cols,
                                                   const uint16_t *__restrict__ x, int B, void *__restrict__ y,
                                                   int out_f32, int RC, int cpw) {
    constexpr int L_ = GEMV_L, STAGE = L_ * 4096;
    static_assert(GEMV_NS == 4, "four stage objects");
    constexpr int PAIR = (DEC == DEC_LUT) ? (FMT == FMT_E2M1 ? LUT_E2M1_PAIR : LUT_E2M3_PAIR) : 1;
    // four stages as separate objects: the compiler can then tell a copy into
    // one stage from reads of another and does not drain the pipeline
    __shared__ __attribute__((aligned(1024))) uint8_t ring0[STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t ring1[STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t ring2[STAGE];
    __shared__ __attribute__((aligned(1024))) uint8_t ring3[STAGE];
    __shared__ u32 s_pair[PAIR];
    __shared__ float s_scale[LUT_SCALE];
    const Luts Lt{s_pair, s_scale};
    const int tid = threadIdx.x;
    build_luts<FMT>(Lt, tid, 256, DEC == DEC_LUT);
    __syncthreads();

    const int crb = (int)Fmt<FMT>::code_row_bytes(cols), srb = (int)Fmt<FMT>::scale_row_bytes(cols);
    const int U = cols / 32, LPR = lanes_per_row(U), RPW = WAVE / LPR;
    const int lane = tid & 63, w = tid >> 6, lr = lane & (LPR - 1), rsub = lane / LPR;
    const __amdgpu_buffer_rsrc_t rc = rsrc_of(codes, (uint64_t)rows * crb);
    const __amdgpu_buffer_rsrc_t rs = rsrc_of(scales, (uint64_t)rows * srb);
    const int NC = (rows + RC - 1) / RC;
    const int c0 = blockIdx.x * cpw;
    const int n = (c0 + cpw < NC ? c0 + cpw : NC) - c0;
    if (n <= 0) return;   // uniform over the workgroup

    auto stage = [&](auto sc) -> uint8_t * {
        constexpr int S = decltype(sc)::value;
        if constexpr (S == 0) return ring0;
        else if constexpr (S == 1) return ring1;
        else if constexpr (S == 2) return ring2;
        else return ring3;
    };
    auto src = [&](int i) {
        const int r0 = (c0 + i) * RC;
        const int nr = (r0 + RC < rows ? r0 + RC : rows) - r0;
        return chunk_src(rc, rs, r0, nr, (u32)crb, (u32)srb);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;

    for (int t0 = 0; t0 < B; t0 += MT) {
        u32 xr[Q][MT][16];
        const uint16_t *xp[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) xp[t] = (t0 + t < B) ? x + (int64_t)(t0 + t) * cols : nullptr;
        load_x_units<Q, MT>(xr, xp, U, lr, LPR);
        wait_vm<0>();   // x in registers before the ring starts

        // chunks 0..2 in flight; chunk i lives in stage i % 4
        issue_chunk<L_>(stage(I0{}), src(0), tid);
        if (1 < n) issue_chunk<L_>(stage(I1{}), src(1), tid);
        if (2 < n) issue_chunk<L_>(stage(I2{}), src(2), tid);

        // Chunk i: wait for this thread's loads of it (loads retire in issue
        // order; chunks i+1, i+2 may still be in flight), barrier (every
        // thread's loads landed, and every wave finished chunk i-1, whose
        // stage the copy of chunk i+3 then reuses), compute.
        auto step = [&](auto dc, int i) {
            constexpr int d = decltype(dc)::value;
            if (i + 2 < n) wait_vm<2 * L_>();
            else if (i + 1 < n) wait_vm<L_>();
            else wait_vm<0>();
            ring_barrier();
            if (i + 3 < n) issue_chunk<L_>(stage(std::integral_constant<int, (d + 3) % 4>{}), src(i + 3), tid);
            const int r0 = (c0 + i) * RC;
            const int nr = (r0 + RC < rows ? r0 + RC : rows) - r0;
            const uint8_t *sc = stage(dc);
            const uint8_t *ss = sc + ((nr * crb + 1023) / 1024) * 1024 + ((r0 * srb) & 15);
            constexpr int R = 2;
            for (int base = w * RPW; base < nr; base += RING_WAVES * RPW * R) {
                int row[R];
#pragma unroll
                for (int b = 0; b < R; ++b) {
                    const int rr = base + b * RING_WAVES * RPW + rsub;
                    row[b] = rr < nr ? rr : -1;
                }
                float acc[R][MT];
                rows_dot_lds<FMT, DEC, Q, MT, R, false>(sc, ss, row, crb, srb, U, lr, LPR, xr, xr, Lt, acc);
#pragma unroll
                for (int b = 0; b < R; ++b) {
                    if (row[b] < 0 || lr != 0) continue;
#pragma unroll
                    for (int t = 0; t < MT; ++t) {
                        if (t0 + t >= B) continue;
                        const int64_t o = (int64_t)(t0 + t) * rows + r0 + row[b];
                        if (out_f32) reinterpret_cast<float *>(y)[o] = acc[b][t];
                        else reinterpret_cast<uint16_t *>(y)[o] = f32_to_bf16_rne(acc[b][t]);
                    }
                }
            }
        };
        for (int i = 0; i < n; i += 4) {
            step(I0{}, i);
            if (i + 1 < n) step(I1{}, i + 1);
            if (i + 2 < n) step(I2{}, i + 2);
            if (i + 3 < n) step(I3{}, i + 3);
        }
        ring_barrier();   // every wave is done with the ring before the next token pass refills it
    }
}

static int num_cus() {
    static int cus = 0;
    if (!cus) {
        int dev = 0;
        (void)hipGetDevice(&dev);
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (cus <= 0) cus = 1;
    }
    return cus;
}

template <int FMT, int DEC, int Q, int MT>
static hipError_t gemv_ring_go(const uint8_t *codes, const uint8_t *scales, int rows, int cols, const uint16_t *x, int B,
                          void *y, int out_f32, hipStream_t s) {
    const int crb = (int)Fmt<FMT>::code_row_bytes(cols), srb = (int)Fmt<FMT>::scale_row_bytes(cols);
    const int RC = rows_per_chunk(GEMV_L, crb, srb);
    const int NC = (rows + RC - 1) / RC;
    const int G0 = num_cus();
    const int cpw = (NC + G0 - 1) / G0;
    const int G = (NC + cpw - 1) / cpw;
    hipLaunchKernelGGL((gemv_ring_kernel<FMT, DEC, Q, MT>), dim3(G), dim3(256), 0, s, codes, scales, rows, cols, x, B, y,
                       out_f32, RC, cpw);
    return hipGetLastError();
}

// Register-streamed variant: the x units stay in VGPRs, and each wave walks
// its rows (every nw-th row group) R per pass with the next pass's loads in
// flight (RowPipe).  A grid of a few workgroups per CU, so every wave streams
// many rows after loading x once.  Used for one token, where it streams
// faster than the ring (fewer VGPRs for x, more waves per CU).
template <int FMT, int DEC, int Q, int MT, int R>
__global__ __launch_bounds__(256) void gemv_reg_kernel(const uint8_t *__restrict__ codes,
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

template <int FMT, int DEC>
static hipError_t gemv_q(const uint8_t *codes, const uint8_t *scales, int rows, int cols, const uint16_t *x, int B,
                         void *y, int out_f32, hipStream_t s) {
    const int U = cols / 32, LPR = lanes_per_row(U), Q = (U + LPR - 1) / LPR;
    const bool one = (B == 1);
#define GO(QQ)                                                                                    \
    if (Q == QQ) {                                                                                \
        if (one) return gemv_reg_go<FMT, DEC, QQ, 1>(codes, scales, rows, cols, x, B, y, out_f32, s); \
        return gemv_ring_go<FMT, DEC, QQ, 4>(codes, scales, rows, cols, x, B, y, out_f32, s);         \
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
