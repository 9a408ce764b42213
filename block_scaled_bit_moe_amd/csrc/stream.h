// stream.h -- streaming block-scaled rows from HBM through an LDS ring.
//
// A workgroup of 4 waves keeps NS chunks of weight rows in flight.  Each chunk
// is one contiguous range of code bytes plus the matching range of scale
// bytes, copied by gfx950's buffer-load-to-LDS (buffer_load_dwordx4 ... lds):
// the data goes from memory straight into LDS without passing through VGPRs,
// so the depth of the pipeline costs LDS, not registers.  Every thread issues
// exactly L 16-byte loads per chunk (pieces beyond the chunk re-load its first
// block into the stage's tail), so a thread can wait for "chunk c landed" with
// one s_waitcnt vmcnt((NS-1)*L): vector-memory loads of a wave return in
// order, and the loads issued after chunk c are exactly the later chunks'.
// Loads go through buffer resources whose range is the matrix, so a read past
// its end returns zeros instead of faulting.
//
// Layout of a stage (L * 4 KiB): codes of rows r0..r0+RC-1 from block 0,
// then (from the next 1 KiB boundary) their scales, whose first byte sits at
// scale_lead = (r0 * scale_row_bytes) % 16 because the copy starts at the
// 16-byte boundary below it.
#pragma once

#include "common.h"

namespace moeq {

constexpr int RING_THREADS = 256;
constexpr int RING_WAVES = 4;
typedef __attribute__((address_space(3))) void lds_void_t;

// The hardware checks the range per dword, so the range is rounded up to the
// 16-byte granule holding the last byte (arrays start 16-byte aligned, so the
// extra bytes never leave that granule, nor its page).
__device__ inline __amdgpu_buffer_rsrc_t rsrc_of(const void *base, uint64_t bytes) {
    bytes = (bytes + 15u) & ~(uint64_t)15u;
    const u32 n = bytes > 0xFFFFFFF0ull ? 0xFFFFFFF0u : (u32)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)n, 0x00020000);
}

struct ChunkSrc {
    __amdgpu_buffer_rsrc_t rc, rs;   // code and scale bytes of the whole matrix
    u32 off_c, blocks_c;             // first code byte (16-aligned), 1 KiB blocks of codes
    u32 off_s, blocks_s;             // first scale byte rounded down to 16, blocks of scales
};

// Describe rows [r0, r0 + nr) of a matrix with crb code / srb scale bytes per row.
__device__ inline ChunkSrc chunk_src(__amdgpu_buffer_rsrc_t rc, __amdgpu_buffer_rsrc_t rs, int r0, int nr,
                                     u32 crb, u32 srb) {
    ChunkSrc c;
    c.rc = rc;
    c.rs = rs;
    c.off_c = (u32)r0 * crb;
    c.blocks_c = ((u32)nr * crb + 1023u) / 1024u;
    const u32 s0 = (u32)r0 * srb;
    c.off_s = s0 & ~15u;
    c.blocks_s = ((s0 & 15u) + (u32)nr * srb + 1023u) / 1024u;
    return c;
}

// Issue the L loads of this thread for one chunk into `stage` (LDS).
template <int L>
__device__ inline void issue_chunk(uint8_t *stage, const ChunkSrc &c, int tid) {
    const int w = tid >> 6, lane = tid & 63;
#pragma unroll
    for (int k = 0; k < L; ++k) {
        const u32 blk = (u32)(k * RING_WAVES + w);
        lds_void_t *dst = (lds_void_t *)(stage + blk * 1024u);
        if (blk < c.blocks_c) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rc, dst, 16, c.off_c + blk * 1024u + lane * 16u, 0, 0, 0);
        } else if (blk < c.blocks_c + c.blocks_s) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rs, dst, 16, c.off_s + (blk - c.blocks_c) * 1024u + lane * 16u,
                                                     0, 0, 0);
        } else {
            // tail: repeat the chunk's first block so every thread issues exactly L loads
            __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rc, dst, 16, c.off_c + lane * 16u, 0, 0, 0);
        }
    }
}

// Wait until this thread's loads of the chunk issued `behind` chunks ago
// have landed (at most `behind` * L later loads still outstanding).
template <int N>
__device__ inline void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Rows that fit in one stage of L * 4 KiB.
__host__ __device__ inline int rows_per_chunk(int L, int crb, int srb) {
    int rc = 1;
    while (true) {
        const int n = rc + 1;
        const int bc = (n * crb + 1023) / 1024, bs = (15 + n * srb + 1023) / 1024;
        if (bc + bs > 4 * L) break;
        rc = n;
    }
    return rc;
}

// One unit of row r of a chunk held in LDS (codes at `codes`, scales at `scales`).
template <int FMT>
__device__ inline void lds_unit(Unit<FMT> &U, const uint8_t *codes, const uint8_t *scales, int r, int crb, int srb,
                                int u) {
    if constexpr (FMT == FMT_E2M1) {
        U.c = *reinterpret_cast<const uint4 *>(codes + r * crb + 16 * u);
        U.s = *reinterpret_cast<const uint16_t *>(scales + r * srb + 2 * u);
    } else {
        const uint8_t *p = codes + r * crb + 24 * u;
        U.c0 = *reinterpret_cast<const uint2 *>(p);
        U.c1 = *reinterpret_cast<const uint2 *>(p + 8);
        U.c2 = *reinterpret_cast<const uint2 *>(p + 16);
        U.s = scales[r * srb + (u >> 2)];
    }
}

// acc[b][t] = row_b . x_t for R rows of a chunk in LDS (row index < 0: skipped,
// result 0).  Same lane mapping, order and reduction as rows_dot.
template <int FMT, int DEC, int Q, int MT, int R, bool SPLIT>
__device__ inline void rows_dot_lds(const uint8_t *codes, const uint8_t *scales, const int (&row)[R], int crb, int srb,
                                    int U, int lr, int LPR, const u32 (&xh)[Q][MT][16], const u32 (&xl)[Q][MT][16],
                                    const Luts &L, float (&acc)[R][MT]) {
    Unit<FMT> un[R][Q];
#pragma unroll
    for (int b = 0; b < R; ++b)
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int u = lr + LPR * q;
            if (u < U && row[b] >= 0) lds_unit<FMT>(un[b][q], codes, scales, row[b], crb, srb, u);
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
            if (u < U && row[b] >= 0) {
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

}  // namespace moeq
