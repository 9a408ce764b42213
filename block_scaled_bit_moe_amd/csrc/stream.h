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
// have landed (at most N loads still outstanding).  Emitted through the
// builtin so that the compiler's own wait insertion knows which loads are
// complete (an s_waitcnt in inline assembly is opaque to it); the clobber
// keeps memory accesses on their side.  Encoding (gfx9): vmcnt in bits 3:0
// and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima.
template <int N>
__device__ inline void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
    asm volatile("" ::: "memory");
}

// Workgroup barrier for the ring.  __syncthreads() carries release/acquire
// fences that make the compiler wait for every outstanding vector load
// (vmcnt(0)), which would empty the ring at each chunk; callers wait for
// exactly the chunk they need with wait_vm first.  The memory clobbers keep
// LDS accesses on their side of the barrier.
__device__ inline void ring_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
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

// LDS reads of the ring in inline assembly.  The compiler cannot always tell
// which stage a pointer inside a loop refers to, and then waits for every
// outstanding buffer-to-LDS copy before each LDS read (vmcnt(0)), which
// empties the ring.  These reads are invisible to that analysis; the
// workgroup barrier after wait_vm already guarantees the chunk has landed,
// and lds_fence() waits for the reads themselves.
typedef __attribute__((ext_vector_type(4))) u32 lds_u32x4;
typedef __attribute__((ext_vector_type(2))) u32 lds_u32x2;
__device__ inline u32 lds_addr(const void *p) {
    return (u32)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}
__device__ inline lds_u32x4 ds_b128(u32 a) {
    lds_u32x4 v;
    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(a));
    return v;
}
__device__ inline lds_u32x2 ds_b64(u32 a) {
    lds_u32x2 v;
    asm volatile("ds_read_b64 %0, %1" : "=v"(v) : "v"(a));
    return v;
}
__device__ inline u32 ds_u8(u32 a) {
    u32 v;
    asm volatile("ds_read_u8 %0, %1" : "=v"(v) : "v"(a));
    return v;
}

// One unit of row r of a chunk held in LDS (codes at `codes`, scales at
// `scales`), read with the assembly loads above: the values are valid only
// after lds_settle().
template <int FMT> struct LdsUnit;
template <> struct LdsUnit<FMT_E2M1> { lds_u32x4 c; u32 s0, s1; };
template <> struct LdsUnit<FMT_E2M3> { lds_u32x2 c0, c1, c2; u32 s; };

template <int FMT>
__device__ inline void lds_unit_issue(LdsUnit<FMT> &V, const uint8_t *codes, const uint8_t *scales, int r, int crb,
                                      int srb, int u) {
    if constexpr (FMT == FMT_E2M1) {
        V.c = ds_b128(lds_addr(codes + r * crb + 16 * u));
        const u32 sa = lds_addr(scales + r * srb + 2 * u);   // any byte alignment
        V.s0 = ds_u8(sa);
        V.s1 = ds_u8(sa + 1);
    } else {
        const u32 p = lds_addr(codes + r * crb + 24 * u);
        V.c0 = ds_b64(p);
        V.c1 = ds_b64(p + 8);
        V.c2 = ds_b64(p + 16);
        V.s = ds_u8(lds_addr(scales + r * srb + (u >> 2)));
    }
}

// Wait for the issued reads, and make every later use of their registers
// depend on that wait.
__device__ inline void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
template <int FMT>
__device__ inline void lds_settle(LdsUnit<FMT> &V, Unit<FMT> &U) {
    if constexpr (FMT == FMT_E2M1) {
        asm volatile("" : "+v"(V.c), "+v"(V.s0), "+v"(V.s1));
        U.c = make_uint4(V.c[0], V.c[1], V.c[2], V.c[3]);
        U.s = V.s0 | (V.s1 << 8);
    } else {
        asm volatile("" : "+v"(V.c0), "+v"(V.c1), "+v"(V.c2), "+v"(V.s));
        U.c0 = make_uint2(V.c0[0], V.c0[1]);
        U.c1 = make_uint2(V.c1[0], V.c1[1]);
        U.c2 = make_uint2(V.c2[0], V.c2[1]);
        U.s = V.s;
    }
}

// acc[b][t] = row_b . x_t for R rows of a chunk in LDS (row index < 0: skipped,
// result 0).  Same lane mapping, order and reduction as rows_dot.
template <int FMT, int DEC, int Q, int MT, int R, bool SPLIT>
__device__ inline void rows_dot_lds(const uint8_t *codes, const uint8_t *scales, const int (&row)[R], int crb, int srb,
                                    int U, int lr, int LPR, const u32 (&xh)[Q][MT][16], const u32 (&xl)[Q][MT][16],
                                    const Luts &L, float (&acc)[R][MT]) {
    Unit<FMT> un[R][Q];
    LdsUnit<FMT> lv[R][Q];
#pragma unroll
    for (int b = 0; b < R; ++b)
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int u = lr + LPR * q;
            // rows past the chunk and units past the row read a valid address; their result is unused
            lds_unit_issue<FMT>(lv[b][q], codes, scales, row[b] >= 0 ? row[b] : 0, crb, srb, u < U ? u : 0);
        }
    lds_wait();
#pragma unroll
    for (int b = 0; b < R; ++b)
#pragma unroll
        for (int q = 0; q < Q; ++q) lds_settle<FMT>(lv[b][q], un[b][q]);
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
