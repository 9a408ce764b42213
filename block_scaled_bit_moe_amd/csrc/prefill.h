// prefill.h -- the MoE layer for many tokens at once, on the matrix cores.
//
// With a prompt chunk of 2,048 tokens and top-10 of 512 experts each expert
// sees about 40 tokens, enough rows for the bf16 matrix instructions to pay
// (knivesysl "Prompt processing" notes; Strata SYCL port, "MoE prefill").
// A chunk runs as five launches on one stream:
//
//   route    top-k per token (the decode path's routing kernel)
//   group    per expert slot, the tokens that selected it in ascending token
//            order; the last workgroup to finish turns the counts into pair
//            offsets and a list of blocks of up to 64 tokens of one slot
//   gate/up  per (block, tile of 64 intermediate rows): g = Wg x, u = Wu x
//            on MFMA 16x16x32 bf16 with fp32 accumulation, then
//            h = silu(g) * u, stored as a bf16 hi + lo pair
//   down     per (block, tile of 512 hidden rows, 256 for six-bit codes): y = Wd (h_hi + h_lo)
//            into fp32 partials, one row per (token, expert) pair
//   combine  per token: sum of w_r * y_r in rank order, plus the shared
//            expert, rounded once to bf16
//
// Weights.  Each wave owns 16-row groups of the weight tile for the whole K
// range, so no other wave needs its decoded weights: a lane loads one unit
// (32 consecutive weights of one row) per 128-wide K step, decodes it with
// the hardware conversion and multiplies in the block scale (exact for the
// minifloat formats: a code value times its scale has at most 8 significant
// bits; int4 times its fp16 scale is carried as two bf16 parts), which gives
// the B operand of four MFMAs directly (pf_unit_to_b).
// Lane l covers row l%16 and the K sub-range 32*(l/16) .. +32 of each step;
// MFMA step s takes weights 8s..8s+7 of that sub-range, so within one
// instruction the four lane groups contribute K offsets {8s, 32+8s, 64+8s,
// 96+8s} + 0..7.  The A operand (token activations) is read with the same
// mapping, so every product pairs a weight with its own activation.
//
// Activations.  The 64 x 128 bf16 activation tile of a K step is staged in
// LDS (row stride 272 bytes, so the 16 rows a quarter-wave reads fall on
// distinct banks), double-buffered, and read by all four waves.
#pragma once

#include <type_traits>

#include "common.h"
#include "memops.h"

namespace moeq {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) u32 u32x4_t;

constexpr int PF_THREADS = 256;
constexpr int PF_MB = 64;                   // tokens per block (four 16-row sub-tiles)
constexpr int PF_KS = 128;                  // K per step
constexpr int PF_ROW = PF_KS * 2 + 16;      // bytes per staged activation row
constexpr int PF_STAGE = PF_MB * PF_ROW;    // bytes per staged plane
constexpr int PF_RG_GU = 1;                 // 16-row groups per wave: gate/up (each of gate and up)
// down: e2m1 takes four (measured: 2 -> 4 took 10 us off the 2,048-token
// layer); six-bit codes' larger units would spill registers with four
template <int FMT> constexpr int pf_rg_dn() { return Fmt<FMT>::SIX ? 2 : 4; }
// int4 weights times their fp16 group scale need up to 14 significant bits, so
// they enter the matrix cores as two bf16 parts, w = hi + lo exactly
template <int FMT> constexpr bool pf_split_w() { return Fmt<FMT>::SCALE == SC_FP16; }
constexpr int PF_PD = 3;                    // weight units in flight per row group (K steps ahead)
constexpr int PF_MAX_K = 32;                // top-k limit of the layer

struct PfArgs {
    LayerArgs L;
    const uint16_t *x;        // bf16 [T][H] of the chunk
    int T;                    // tokens in the chunk
    int NS;                   // expert slots: E routed, +1 shared (slot E)
    int mode, fixed_e;
    const int32_t *idx;       // [T][k] (route mode)
    const float *w;           // [T][k]
    int32_t *rank;            // [T][k]: position of the token in its expert's list
    int32_t *cnt;             // [NS]
    int32_t *off;             // [NS + 1]: first pair of each slot
    int32_t *nblk;            // [1]
    int32_t *blk;             // [nblk_max]: slot << 16 | first token of the block
    int32_t *tok;             // [NS][T]: token ids of each slot, ascending
    uint16_t *h_hi, *h_lo;    // [pairs][Imax] bf16
    float *y;                 // [pairs][H] fp32
    void *out;                // [T][H] bf16 or fp32
    int out_f32;
    const uint16_t *residual; // bf16 [T][H] of the chunk added before rounding (nullable)
    uint32_t *hdr;            // workspace header (arrival counter)
    int Imax;
    const uint8_t *xq;        // MX e4m3 activations [T][H] of the chunk (scaled matrix cores; nullable)
    const uint8_t *xs;        // their UE8M0 scales [T][H/32]
};

constexpr int WS_PF_ARRIVE = 4;   // header word: group workgroups finished

__device__ inline void pf_st_relaxed(int32_t *p, int32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline int32_t pf_ld_relaxed(const int32_t *p) {
    return __hip_atomic_load(const_cast<int32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Which slot receives which tokens.  In route mode slot e < E gets the tokens
// whose top-k holds e and slot E (the shared expert) every token; with a
// fixed expert only that slot is active and it gets every token.
__device__ inline bool pf_slot_identity(const PfArgs &a, int slot) {
    if (a.mode == MODE_ROUTE) return slot == a.L.E;
    return a.mode == MODE_FIXED_ROUTED ? slot == a.fixed_e : slot == a.L.E;
}

// Exclusive scan over the 256 threads of a block (values in v, total returned).
__device__ inline int pf_block_scan(int v, int *s_tmp, int tid, int &total) {
    const int lane = tid & 63, wv = tid >> 6;
    // inclusive scan within the wave
    int x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    if (lane == 63) s_tmp[wv] = x;
    __syncthreads();
    int base = 0;
    for (int i = 0; i < wv; ++i) base += s_tmp[i];
    total = s_tmp[0] + s_tmp[1] + s_tmp[2] + s_tmp[3];
    __syncthreads();
    return base + x - v;
}

__global__ __launch_bounds__(PF_THREADS) void pf_group_kernel(PfArgs a) {
    const int slot = blockIdx.x, tid = threadIdx.x;
    const int T = a.T, k = a.L.k;
    __shared__ int s_tmp[4];
    __shared__ int s_last;
    int count = 0;
    int32_t *list = a.tok + (size_t)slot * T;
    if (pf_slot_identity(a, slot)) {
        for (int t = tid; t < T; t += PF_THREADS) list[t] = t;
        count = T;
    } else if (a.mode == MODE_ROUTE) {
        // Wave w scans the index words of tokens [w * span, (w + 1) * span),
        // 64 consecutive words per load (coalesced, 16 loads in flight); a word equal to this slot
        // is the hit of token word / k at rank word % k (a token picks a slot
        // at most once), and the words are in token order, so a ballot gives
        // each hit its place among the wave's hits.  Pass 1 counts, one
        // barrier gives the four waves' bases, pass 2 (the words again, from
        // L2) writes the list in ascending token order.
        const int wv = tid >> 6, lane = tid & 63;
        const int span = (T + 3) / 4;
        const int d0 = min(T, wv * span) * k, d1 = min(T, (wv + 1) * span) * k;
        constexpr int UNR = 16;   // loads in flight per lane
        int mine = 0;
        for (int d = d0; d < d1; d += 64 * UNR) {
            int v[UNR];
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                const int dd = d + 64 * u + lane;
                v[u] = dd < d1 ? a.idx[dd] : -1;
            }
#pragma unroll
            for (int u = 0; u < UNR; ++u) mine += __popcll(__ballot(v[u] == slot));
        }
        if (lane == 0) s_tmp[wv] = mine;
        __syncthreads();
        int pos = 0;
        for (int w = 0; w < wv; ++w) pos += s_tmp[w];
        count = s_tmp[0] + s_tmp[1] + s_tmp[2] + s_tmp[3];
        for (int d = d0; d < d1; d += 64 * UNR) {
            int v[UNR];
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                const int dd = d + 64 * u + lane;
                v[u] = dd < d1 ? a.idx[dd] : -1;
            }
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                const uint64_t hit = __ballot(v[u] == slot);
                if (v[u] == slot) {
                    const int dd = d + 64 * u + lane;
                    const int t = dd / k, r = dd - t * k;
                    const int p = pos + (int)__popcll(hit & ((1ull << lane) - 1ull));
                    list[p] = t;
                    a.rank[(size_t)t * k + r] = p;
                }
                pos += (int)__popcll(hit);
            }
        }
    }
    // publish the count; the last workgroup to arrive builds the plan
    if (tid == 0) {
        pf_st_relaxed(&a.cnt[slot], count);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        const u32 prev = __hip_atomic_fetch_add(&a.hdr[WS_PF_ARRIVE], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (prev == (u32)(a.NS - 1)) ? 1 : 0;
    }
    __syncthreads();
    if (!s_last) return;
    // plan: pair offsets and the block list, slot by slot in ascending order
    const int NS = a.NS;
    const int per = (NS + PF_THREADS - 1) / PF_THREADS;
    const int s0 = tid * per;
    int c_sum = 0, b_sum = 0;
    for (int s = s0; s < s0 + per && s < NS; ++s) {
        const int c = pf_ld_relaxed(&a.cnt[s]);
        c_sum += c;
        b_sum += (c + PF_MB - 1) / PF_MB;
    }
    int c_tot, b_tot;
    int c_base = pf_block_scan(c_sum, s_tmp, tid, c_tot);
    int b_base = pf_block_scan(b_sum, s_tmp, tid, b_tot);
    for (int s = s0; s < s0 + per && s < NS; ++s) {
        const int c = pf_ld_relaxed(&a.cnt[s]);
        a.off[s] = c_base;
        const int nb = (c + PF_MB - 1) / PF_MB;
        for (int j = 0; j < nb; ++j) a.blk[b_base + j] = (s << 16) | (j * PF_MB);
        c_base += c;
        b_base += nb;
    }
    if (tid == 0) {
        a.off[NS] = c_tot;
        a.nblk[0] = b_tot;
        __hip_atomic_store(&a.hdr[WS_PF_ARRIVE], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Weight units of one K step for the NB row groups of a lane.  Addresses are
// clamped into the row so the loads need no branch (the compiler can then
// count outstanding loads exactly); units past the row's end are zeroed at
// conversion.
template <int FMT>
__device__ inline Unit<FMT> pf_load_unit(const uint8_t *rc, const uint8_t *rs, int u) {
    Unit<FMT> U;
    load_unit<FMT>(U, rc, rs, u);
    return U;
}

// Decode one unit, block scale included, into the B operands of the four MFMA
// steps of a K step (step s takes weights 8s .. 8s+7 of the unit).
//  e2m1 + e4m3 and e2m3 + e4m3: codes -> fp32, times the scale of their block
//    of 16 (exact: a code value has at most 4 significant bits and an e4m3
//    scale 4, and the product stays inside bf16's range), packed to bf16;
//  e2m3 + UE8M0 and e2m1 + UE8M0: the conversion applies the power-of-two
//    scale itself (it takes the scale's exponent field, which is all a UE8M0
//    scale has): exact while code value times scale stays inside bf16's range;
//  int4 + fp16: w = code * scale is exact in fp32 but needs up to 14 bits, so
//    it is split into bf16 hi = RNE(w) and lo = w - hi (exact, at most 7 bits)
//    and the matrix cores take both (b and bl).
__device__ inline u32 pf_pack2(float a, float b) { return __builtin_bit_cast(u32, bf16x2_t{(__bf16)a, (__bf16)b}); }

template <int FMT>
__device__ inline void pf_unit_to_b(const Unit<FMT> &U, const float *s_scale, bf16x8_t (&b)[4], bf16x8_t (&bl)[4]) {
    using F = Fmt<FMT>;
    if constexpr (FMT == FMT_E2M1) {
        const float s0 = s_scale[U.s & 0xFF], s1 = s_scale[(U.s >> 8) & 0xFF];
        const u32 d[4] = {U.c.x, U.c.y, U.c.z, U.c.w};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const float sc = s < 2 ? s0 : s1;
            const f2_t f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d[s], 1.0f, 0);
            const f2_t f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d[s], 1.0f, 1);
            const f2_t f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d[s], 1.0f, 2);
            const f2_t f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d[s], 1.0f, 3);
            u32x4_t v;
            v[0] = pf_pack2(f0.x * sc, f0.y * sc);
            v[1] = pf_pack2(f1.x * sc, f1.y * sc);
            v[2] = pf_pack2(f2.x * sc, f2.y * sc);
            v[3] = pf_pack2(f3.x * sc, f3.y * sc);
            b[s] = __builtin_bit_cast(bf16x8_t, v);
        }
    } else if constexpr (FMT == FMT_MXFP4) {
        const float sc = __builtin_bit_cast(float, (U.s & 0xFFu) << 23);
        const u32 d[4] = {U.c.x, U.c.y, U.c.z, U.c.w};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            u32x4_t v;
            v[0] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[s], sc, 0));
            v[1] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[s], sc, 1));
            v[2] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[s], sc, 2));
            v[3] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[s], sc, 3));
            b[s] = __builtin_bit_cast(bf16x8_t, v);
        }
    } else if constexpr (FMT == FMT_INT4) {
        const float sc = (float)__builtin_bit_cast(_Float16, (uint16_t)(U.s & 0xFFFF));
        const u32 d[4] = {U.c.x, U.c.y, U.c.z, U.c.w};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            u32x4_t vh, vl;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float w0 = (float)(((int)(d[s] << (28 - 8 * q))) >> 28) * sc;
                const float w1 = (float)(((int)(d[s] << (24 - 8 * q))) >> 28) * sc;
                const u32 h = pf_pack2(w0, w1);
                vh[q] = h;
                vl[q] = pf_pack2(w0 - __builtin_bit_cast(float, h << 16), w1 - __builtin_bit_cast(float, h & 0xFFFF0000u));
            }
            b[s] = __builtin_bit_cast(bf16x8_t, vh);
            bl[s] = __builtin_bit_cast(bf16x8_t, vl);
        }
    } else if constexpr (FMT == FMT_E2M3S) {
        u32x6_t v;
        v[0] = U.c0.x; v[1] = U.c0.y; v[2] = U.c1.x; v[3] = U.c1.y; v[4] = U.c2.x; v[5] = U.c2.y;
        typedef __attribute__((ext_vector_type(32))) float f32x32_t;
        const f32x32_t f = __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(v, 1.0f);
        const float s0 = s_scale[U.s & 0xFF], s1 = s_scale[(U.s >> 8) & 0xFF];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const float sc = s < 2 ? s0 : s1;
            u32x4_t q4;
#pragma unroll
            for (int q = 0; q < 4; ++q) q4[q] = pf_pack2(f[8 * s + 2 * q] * sc, f[8 * s + 2 * q + 1] * sc);
            b[s] = __builtin_bit_cast(bf16x8_t, q4);
        }
    } else {
        static_assert(FMT == FMT_E2M3, "format");
        u32x6_t v;
        v[0] = U.c0.x; v[1] = U.c0.y; v[2] = U.c1.x; v[3] = U.c1.y; v[4] = U.c2.x; v[5] = U.c2.y;
        const float sc = __builtin_bit_cast(float, (U.s & 0xFFu) << 23);
        const bf16x32_t r = __builtin_amdgcn_cvt_scalef32_pk32_bf16_fp6(v, sc);
        typedef __attribute__((ext_vector_type(16))) u32 u32x16_t;
        const u32x16_t rr = __builtin_bit_cast(u32x16_t, r);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            u32x4_t q;
            q[0] = rr[4 * s]; q[1] = rr[4 * s + 1]; q[2] = rr[4 * s + 2]; q[3] = rr[4 * s + 3];
            b[s] = __builtin_bit_cast(bf16x8_t, q);
        }
    }
    (void)F::SIX;
}

template <int FMT>
__device__ inline void pf_zero_unit(Unit<FMT> &U) {
    if constexpr (!Fmt<FMT>::SIX) {
        U.c = make_uint4(0u, 0u, 0u, 0u);
    } else {
        U.c0 = make_uint2(0u, 0u);
        U.c1 = U.c0;
        U.c2 = U.c0;
    }
    U.s = 0u;
}

// Barrier without the release/acquire fences of __syncthreads(): those make
// the compiler drain every outstanding vector load (vmcnt(0)), which would
// empty the prefetch pipeline at each step.  Callers wait for exactly the
// loads they need first; the memory clobbers keep the compiler from moving
// LDS accesses across the barrier.
__device__ inline void pf_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <int N>
__device__ inline void pf_wait_vm() {
    wait_vm<N>();
}

// Vector-memory loads of one weight unit.
template <int FMT> struct PfUnitLoads { static constexpr int n = Fmt<FMT>::SIX ? 4 : 2; };

// Grouped GEMM main loop for a block of NSUB 16-token sub-tiles.
//
// Pipeline.  K step j needs (i) the activation tile of step j, copied from
// HBM/L2 straight into an LDS stage by buffer-load-to-LDS, and (ii) each
// lane's weight units of step j, in registers.  Both are issued together, PD
// steps ahead, into a ring of PD + 1 LDS stages and PD register slots.
// Vector-memory loads of a wave complete in issue order, so "step j landed"
// is one s_waitcnt vmcnt(loads issued after step j's group); the barrier
// that follows makes every wave's copy of stage j visible, and since the
// next copy is issued after that barrier it only overwrites the stage all
// waves finished reading one step earlier.
//
// Activation stage layout: plane pl (x, or h_hi / h_lo), rows 16 * NSUB of
// 256 bytes (128 bf16); the 16-byte piece c of row r sits at c ^ (r & 15), so
// the 16 rows a quarter-wave reads for one MFMA hit 16 different bank groups.
template <int FMT, bool DOWN, int NSUB, int NWAVES, int RG>
__device__ inline void pf_gemm_main(const PfArgs &a, uint8_t *st0, uint8_t *st1, uint8_t *st2, uint8_t *st3,
                                    const float *s_scale, const int *s_tok, int M,
                                    int p0, int K, int N, int n0, const uint8_t *const (&rc)[DOWN ? RG : 2 * RG],
                                    const uint8_t *const (&rs)[DOWN ? RG : 2 * RG]) {
    constexpr int NB = DOWN ? RG : 2 * RG;
    constexpr int NPL = DOWN ? 2 : 1;
    constexpr int PLANE = NSUB * 16 * 256;                  // bytes per plane of a stage
    constexpr int R = PF_PD + 1;                            // stages in the ring (separate LDS objects)
    static_assert(R == 4, "four stage objects");
    constexpr int NDMA = NSUB * 4 * NPL;                    // 1 KiB copies per stage
    static_assert(NDMA % NWAVES == 0, "copies per wave");
    constexpr int DPW = NDMA / NWAVES;                      // per wave
    constexpr int PER_GROUP = DPW + NB * PfUnitLoads<FMT>::n;   // loads a wave issues per step
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int lg = lane >> 4, lr = lane & 15;
    const int H = a.L.H;
    const int nK = (K + PF_KS - 1) / PF_KS;
    const int UK = K / 32;

    // the activation copies of this lane: byte offset of its row's first
    // element (plus its piece's column) in the source buffer
    __amdgpu_buffer_rsrc_t src[NPL];
    if (DOWN) {
        const uint64_t bytes = (uint64_t)a.off[a.NS] * a.Imax * 2;
        src[0] = rsrc_of(a.h_hi, bytes);
        src[NPL - 1] = rsrc_of(a.h_lo, bytes);
    } else {
        src[0] = rsrc_of(a.x, (uint64_t)a.T * H * 2);
    }
    u32 row_off[DPW], col_k[DPW];
    int dst_off[DPW], dpl[DPW];
#pragma unroll
    for (int q = 0; q < DPW; ++q) {
        const int g = q * NWAVES + wv;                      // copy index in the stage
        const int pl = g / (NSUB * 4);
        const int P = (g % (NSUB * 4)) * 64 + lane;         // 16-byte piece of the plane
        const int row = P >> 4;
        const int logical = (P & 15) ^ (row & 15);
        const int rr = min(row, M - 1);
        row_off[q] = DOWN ? (u32)(p0 + rr) * (u32)a.Imax * 2u : (u32)s_tok[rr] * (u32)H * 2u;
        col_k[q] = (u32)logical * 8u;
        dst_off[q] = pl * PLANE + (g % (NSUB * 4)) * 1024;
        dpl[q] = pl;
    }
    // stage S of the ring; distinct objects, so the compiler can tell a copy
    // into one stage from reads of another and need not wait between them
    auto stage = [&](auto sc) -> uint8_t * {
        constexpr int S = decltype(sc)::value;
        if constexpr (S == 0) return st0;
        else if constexpr (S == 1) return st1;
        else if constexpr (S == 2) return st2;
        else return st3;
    };
    auto issue_stage = [&](auto sc, int j) {
        uint8_t *st = stage(sc);
        const u32 kb = (u32)j * PF_KS;
#pragma unroll
        for (int q = 0; q < DPW; ++q) {
            const u32 k = kb + col_k[q];
            const u32 voff = k < (u32)K ? row_off[q] + k * 2u : 0x7FFFFFF0u;   // past K: reads as zeros
            __builtin_amdgcn_raw_ptr_buffer_load_lds(src[dpl[q]], (lds_void_t *)(st + dst_off[q]), 16, voff, 0, 0, 0);
        }
    };

    Unit<FMT> wq[R][NB];
    auto load_w = [&](Unit<FMT> (&U)[NB], int j) {
        const int u = min(j * 4 + lg, UK - 1);              // clamped: no branch, result unused past the end
#pragma unroll
        for (int b = 0; b < NB; ++b) load_unit<FMT>(U[b], rc[b], rs[b], u);
    };

    f32x4_t acc[NB][NSUB];
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int m = 0; m < NSUB; ++m) acc[j][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    // prologue: steps 0 .. PD-1 in flight
    issue_stage(I0{}, 0);
    load_w(wq[0], 0);
    issue_stage(I1{}, 1);
    load_w(wq[1], 1);
    issue_stage(I2{}, 2);
    load_w(wq[2], 2);

    // step it uses stage and weight slot it % 4 and refills slot (it + 3) % 4
    auto step = [&](auto dc, int it) {
        constexpr int d = decltype(dc)::value;
        constexpr int dn = (d + PF_PD) % R;
        pf_wait_vm<(PF_PD - 1) * PER_GROUP>();              // this wave's step-it loads have landed
        pf_barrier();                                       // ... and every wave's; stage (it-1) % R is free
        if (it * 4 + lg >= UK) {                            // units past the row's end: zero weights
#pragma unroll
            for (int j = 0; j < NB; ++j) pf_zero_unit<FMT>(wq[d][j]);
        }
        constexpr bool WLO = pf_split_w<FMT>();
        bf16x8_t bw[NB][4], bwl[NB][4];
#pragma unroll
        for (int j = 0; j < NB; ++j) pf_unit_to_b<FMT>(wq[d][j], s_scale, bw[j], bwl[j]);
        issue_stage(std::integral_constant<int, dn>{}, it + PF_PD);
        load_w(wq[dn], it + PF_PD);
        const uint8_t *st = stage(dc);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int piece = ((lg * 4 + s) ^ lr) * 16;
            bf16x8_t ah[NSUB], al[NSUB];
#pragma unroll
            for (int m = 0; m < NSUB; ++m) {
                const uint8_t *ap = st + (16 * m + lr) * 256 + piece;
                ah[m] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t *>(ap));
                if (DOWN) al[m] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t *>(ap + PLANE));
            }
#pragma unroll
            for (int m = 0; m < NSUB; ++m)
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    acc[j][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[m], bw[j][s], acc[j][m], 0, 0, 0);
                    if (DOWN)
                        acc[j][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[m], bw[j][s], acc[j][m], 0, 0, 0);
                    if (WLO) {
                        acc[j][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[m], bwl[j][s], acc[j][m], 0, 0, 0);
                        if (DOWN)
                            acc[j][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[m], bwl[j][s], acc[j][m], 0, 0, 0);
                    }
                }
        }
    };
    int it = 0;
    for (; it + R <= nK; it += R) {
        step(I0{}, it);
        step(I1{}, it + 1);
        step(I2{}, it + 2);
        step(I3{}, it + 3);
    }
    if (it < nK) step(I0{}, it);
    if (it + 1 < nK) step(I1{}, it + 1);
    if (it + 2 < nK) step(I2{}, it + 2);
    // drain the copies issued past the end before the workgroup's LDS is reused
    pf_wait_vm<0>();

    // epilogue: lane holds rows (tokens) 16m + 4 lg + i, column (weight row) lr
#pragma unroll
    for (int g = 0; g < RG; ++g) {
        const int n = n0 + wv * 16 * RG + g * 16 + lr;
        if (n >= N) continue;
#pragma unroll
        for (int m = 0; m < NSUB; ++m) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * m + 4 * lg + i;
                if (t >= M) continue;
                const size_t p = (size_t)(p0 + t);
                if (DOWN) {
                    a.y[p * H + n] = acc[g][m][i];
                } else {
                    const float h = silu_f32(acc[g][m][i]) * acc[RG + g][m][i];
                    const uint16_t hi = f32_to_bf16_rne(h);
                    const uint16_t lo = f32_to_bf16_rne(h - __builtin_bit_cast(float, (u32)hi << 16));
                    a.h_hi[p * a.Imax + n] = hi;
                    a.h_lo[p * a.Imax + n] = lo;
                }
            }
        }
    }
}

// Grouped GEMM over the block list.  gate/up (DOWN = false): 4 waves, each
// with 16 rows of gate and the same 16 rows of up; down: 8 waves of 64 rows
// (four-bit codes) or 32 rows (six-bit codes).
template <int FMT, bool DOWN>
__global__ __launch_bounds__(DOWN ? 512 : 256, DOWN ? 1 : 2) void pf_gemm_kernel(PfArgs a, int NT) {
    constexpr int NWAVES = DOWN ? 8 : 4;
    constexpr int RG = DOWN ? pf_rg_dn<FMT>() : PF_RG_GU;
    constexpr int NB = DOWN ? RG : 2 * RG;
    constexpr int NPL = DOWN ? 2 : 1;
    constexpr int ROWS_WG = NWAVES * 16 * RG;
    constexpr int STAGE_BYTES = NPL * 4 * 16 * 256;
    __shared__ __attribute__((aligned(1024))) uint8_t pf_st0[STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t pf_st1[STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t pf_st2[STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t pf_st3[STAGE_BYTES];
    __shared__ float s_scale[LUT_SCALE];
    __shared__ int s_tok[PF_MB];

    // block and tile of this workgroup; the NT tiles of a block share an XCD
    const int wid = blockIdx.x;
    const int win = wid / (8 * NT), q = wid - win * 8 * NT;
    const int b = win * 8 + (q & 7), nt = q >> 3;
    if (b >= a.nblk[0]) return;
    const int packed = a.blk[b];
    const int slot = packed >> 16, m0 = packed & 0xFFFF;
    const int E = a.L.E, H = a.L.H;
    const bool shared = slot == E;
    const int Is = shared ? a.L.Ish : a.L.I;
    const int N = DOWN ? H : Is;
    const int K = DOWN ? Is : H;
    const int n0 = nt * ROWS_WG;
    if (n0 >= N) return;
    const int M = min(PF_MB, a.cnt[slot] - m0);
    const int nsub = (M + 15) >> 4;
    const int p0 = a.off[slot] + m0;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int lr = lane & 15;

    if (Fmt<FMT>::SCALE == SC_E4M3) {   // the other scales are converted arithmetically
        Luts Lt;
        Lt.pair = nullptr;
        Lt.scale = s_scale;
        build_luts<FMT>(Lt, tid, NWAVES * 64, false);
    }
    if (!DOWN && tid < PF_MB) s_tok[tid] = a.tok[(size_t)slot * a.T + m0 + min(tid, M - 1)];

    // weight rows of this wave
    using F = Fmt<FMT>;
    const int64_t crb = F::code_row_bytes(K), srb = F::scale_row_bytes(K);
    const uint8_t *wc, *ws;
    if (DOWN) {
        wc = shared ? a.L.sh2c : a.L.w2c + (size_t)slot * H * crb;
        ws = shared ? a.L.sh2s : a.L.w2s + (size_t)slot * H * srb;
    } else {
        wc = shared ? a.L.sh13c : a.L.w13c + (size_t)slot * 2 * Is * crb;
        ws = shared ? a.L.sh13s : a.L.w13s + (size_t)slot * 2 * Is * srb;
    }
    const uint8_t *rc[NB];
    const uint8_t *rs[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
        const int g = DOWN ? j : (j % RG);
        const int n = min(n0 + wv * 16 * RG + g * 16 + lr, N - 1);   // rows past N: a valid row, result dropped
        const int row = (!DOWN && j >= RG) ? Is + n : n;
        rc[j] = wc + (size_t)row * crb;
        rs[j] = ws + (size_t)row * srb;
    }
    __syncthreads();   // s_tok, scale table
    switch (nsub) {
        case 1: pf_gemm_main<FMT, DOWN, 1, NWAVES, RG>(a, pf_st0, pf_st1, pf_st2, pf_st3, s_scale, s_tok, M, p0, K, N, n0, rc, rs); break;
        case 2: pf_gemm_main<FMT, DOWN, 2, NWAVES, RG>(a, pf_st0, pf_st1, pf_st2, pf_st3, s_scale, s_tok, M, p0, K, N, n0, rc, rs); break;
        case 3: pf_gemm_main<FMT, DOWN, 3, NWAVES, RG>(a, pf_st0, pf_st1, pf_st2, pf_st3, s_scale, s_tok, M, p0, K, N, n0, rc, rs); break;
        default: pf_gemm_main<FMT, DOWN, 4, NWAVES, RG>(a, pf_st0, pf_st1, pf_st2, pf_st3, s_scale, s_tok, M, p0, K, N, n0, rc, rs); break;
    }
}

// Gate | up on the scaled matrix cores for the MX weight formats (e2m1 or
// e2m3 codes with UE8M0 scales per 32, or per 128 = four blocks of 32 with one
// byte) and MX e4m3 activations (scale per 32): v_mfma_scale_f32_16x16x128_f8f6f4
// with the activations as A (16 tokens) and the weights as B (16 rows).  The
// operand layout of that instruction, measured on this part with one-hot and
// random operands: B lane group h holds K 32h .. 32h+31 of its column; A lane
// group g holds K 16g .. 16g+15 in its first 16 bytes and 64+16g .. 64+16g+15
// in its last 16; the scale of K block b (K 32b .. 32b+31) is lane group b's
// scale byte, for A and for B alike, whichever lanes hold that block's data.
// So for the 128-wide K step s, B lane group h loads weight unit 4s + h with
// its scale, and A lane group g loads its two 16-byte pieces of the token's
// codes and the scale of activation block 4s + g: one instruction per step.
// One workgroup per (block of 64 tokens, tile of 64 intermediate rows), four
// waves of 16 gate and the same 16 up rows; the next K step's loads are issued
// before this step's MFMAs.  The epilogue is the bf16 path's: h = silu(g) * u
// as a bf16 hi + lo pair.
typedef __attribute__((ext_vector_type(8))) int v8i_t;

template <int FMT>
__device__ inline v8i_t pf_mx_b(const Unit<FMT> &U) {
    v8i_t v = {0, 0, 0, 0, 0, 0, 0, 0};
    if constexpr (!Fmt<FMT>::SIX) {
        v[0] = (int)U.c.x; v[1] = (int)U.c.y; v[2] = (int)U.c.z; v[3] = (int)U.c.w;
    } else {
        v[0] = (int)U.c0.x; v[1] = (int)U.c0.y; v[2] = (int)U.c1.x; v[3] = (int)U.c1.y; v[4] = (int)U.c2.x;
        v[5] = (int)U.c2.y;
    }
    return v;
}

template <int FMT>
__global__ __launch_bounds__(256) void pf_gateup_mx_kernel(PfArgs a, int NT) {
    static_assert(Fmt<FMT>::SCALE == SC_UE8M0, "MX weight formats only");
    constexpr int BFMT = Fmt<FMT>::SIX ? 2 : 4;        // fp6 e2m3 or fp4 e2m1 operand
    __shared__ int s_tok[PF_MB];
    const int wid = blockIdx.x;
    const int win = wid / (8 * NT), q = wid - win * 8 * NT;
    const int b = win * 8 + (q & 7), nt = q >> 3;
    if (b >= a.nblk[0]) return;
    const int packed = a.blk[b];
    const int slot = packed >> 16, m0 = packed & 0xFFFF;
    const int E = a.L.E, H = a.L.H;
    const bool shared = slot == E;
    const int Is = shared ? a.L.Ish : a.L.I;
    const int n0 = nt * 64;
    if (n0 >= Is) return;
    const int M = min(PF_MB, a.cnt[slot] - m0);
    const int p0 = a.off[slot] + m0;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    if (tid < PF_MB) s_tok[tid] = a.tok[(size_t)slot * a.T + m0 + min(tid, M - 1)];
    __syncthreads();

    using F = Fmt<FMT>;
    const int64_t crb = F::code_row_bytes(H), srb = F::scale_row_bytes(H);
    const uint8_t *wc = shared ? a.L.sh13c : a.L.w13c + (size_t)slot * 2 * Is * crb;
    const uint8_t *ws = shared ? a.L.sh13s : a.L.w13s + (size_t)slot * 2 * Is * srb;
    const int n = min(n0 + wv * 16 + lr, Is - 1);     // rows past Is: a valid row, result dropped
    const uint8_t *rc[2] = {wc + (size_t)n * crb, wc + (size_t)(Is + n) * crb};
    const uint8_t *rs[2] = {ws + (size_t)n * srb, ws + (size_t)(Is + n) * srb};
    const int UK = H / 32, nK = (H + 127) / 128, HB = H / 32;
    const uint8_t *arow[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) arow[m] = a.xq + (size_t)s_tok[min(16 * m + lr, M - 1)] * H;
    const uint8_t *srow[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) srow[m] = a.xs + (size_t)s_tok[min(16 * m + lr, M - 1)] * HB;
    const int nsub = (M + 15) >> 4;

    Unit<FMT> wu[2][2];
    uint4 ax[2][4][2];
    u32 as[2][4];
    auto load = [&](int st, int j) {
        const int u = min(j * 4 + lg, UK - 1);
#pragma unroll
        for (int g = 0; g < 2; ++g) load_unit<FMT>(wu[st][g], rc[g], rs[g], u);
        // the two activation pieces, K 128 j + 16 lg and 128 j + 64 + 16 lg (kept inside the row)
        const int k0 = min(128 * j + 16 * lg, H - 16), k1 = min(128 * j + 64 + 16 * lg, H - 16);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            ax[st][m][0] = *reinterpret_cast<const uint4 *>(arow[m] + k0);
            ax[st][m][1] = *reinterpret_cast<const uint4 *>(arow[m] + k1);
            as[st][m] = srow[m][u];
        }
    };
    f32x4_t acc[2][4];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int m = 0; m < 4; ++m) acc[g][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    auto step = [&](int st, int j) {
        // K blocks past the row's end: weights 0 with unit scales, so they add exactly 0
        const bool live = j * 4 + lg < UK;
        v8i_t bw[2];
        int bs[2];
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            bw[g] = live ? pf_mx_b<FMT>(wu[st][g]) : v8i_t{0, 0, 0, 0, 0, 0, 0, 0};
            bs[g] = live ? (int)(wu[st][g].s & 0xFF) : 127;
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            if (m < nsub) {
                const v8i_t av = {(int)ax[st][m][0].x, (int)ax[st][m][0].y, (int)ax[st][m][0].z, (int)ax[st][m][0].w,
                                  (int)ax[st][m][1].x, (int)ax[st][m][1].y, (int)ax[st][m][1].z, (int)ax[st][m][1].w};
                const int sa = live ? (int)as[st][m] : 127;
#pragma unroll
                for (int g = 0; g < 2; ++g)
                    acc[g][m] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bw[g], acc[g][m], 0, BFMT, 0, sa, 0,
                                                                                 bs[g]);
            }
        }
    };
    load(0, 0);
    for (int j = 0; j < nK; j += 2) {
        load(1, j + 1);
        step(0, j);
        if (j + 1 >= nK) break;
        load(0, j + 2);
        step(1, j + 1);
    }
    // epilogue: lane holds tokens 16m + 4 lg + i, weight row n0 + 16 wv + lr
    const int nn = n0 + wv * 16 + lr;
    if (nn >= Is) return;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 16 * m + 4 * lg + i;
            if (t >= M) continue;
            const size_t p = (size_t)(p0 + t);
            const float h = silu_f32(acc[0][m][i]) * acc[1][m][i];
            const uint16_t hi = f32_to_bf16_rne(h);
            const uint16_t lo = f32_to_bf16_rne(h - __builtin_bit_cast(float, (u32)hi << 16));
            a.h_hi[p * a.Imax + nn] = hi;
            a.h_lo[p * a.Imax + nn] = lo;
        }
    }
}

// out[t] = sum_r w[t][r] * y[pair(t, r)] (rank order) + y[shared pair of t];
// with a fixed expert, out[t] = y[pair of t].
__global__ __launch_bounds__(PF_THREADS) void pf_combine_kernel(PfArgs a) {
    const int t = blockIdx.x, tid = threadIdx.x;
    const int H = a.L.H, k = a.L.k, E = a.L.E;
    __shared__ int s_p[PF_MAX_K + 1];
    __shared__ float s_w[PF_MAX_K];
    int np = 0;
    bool add_shared = false;
    if (a.mode == MODE_ROUTE) {
        if (tid < k) {
            const int e = a.idx[(size_t)t * k + tid];
            s_p[tid] = a.off[e] + a.rank[(size_t)t * k + tid];
            s_w[tid] = a.w[(size_t)t * k + tid];
        }
        if (tid == 0 && a.L.Ish > 0) s_p[k] = a.off[E] + t;
        np = k;
        add_shared = a.L.Ish > 0;
    } else {
        const int slot = a.mode == MODE_FIXED_ROUTED ? a.fixed_e : E;
        if (tid == 0) s_p[0] = a.off[slot] + t;
    }
    __syncthreads();
    for (int c = tid * 4; c < H; c += PF_THREADS * 4) {
        float4 acc;
        if (a.mode == MODE_ROUTE) {
            acc = make_float4(0.f, 0.f, 0.f, 0.f);
            for (int r = 0; r < np; ++r) {
                const float4 v = *reinterpret_cast<const float4 *>(a.y + (size_t)s_p[r] * H + c);
                const float wr = s_w[r];
                acc.x = __builtin_fmaf(wr, v.x, acc.x);
                acc.y = __builtin_fmaf(wr, v.y, acc.y);
                acc.z = __builtin_fmaf(wr, v.z, acc.z);
                acc.w = __builtin_fmaf(wr, v.w, acc.w);
            }
            if (add_shared) {
                const float4 v = *reinterpret_cast<const float4 *>(a.y + (size_t)s_p[k] * H + c);
                acc.x += v.x;
                acc.y += v.y;
                acc.z += v.z;
                acc.w += v.w;
            }
        } else {
            acc = *reinterpret_cast<const float4 *>(a.y + (size_t)s_p[0] * H + c);
        }
        const size_t o = (size_t)t * H + c;
        if (a.residual) {
            const uint2 r = *reinterpret_cast<const uint2 *>(a.residual + o);
            acc.x += bf16_to_f32((uint16_t)(r.x & 0xFFFF));
            acc.y += bf16_to_f32((uint16_t)(r.x >> 16));
            acc.z += bf16_to_f32((uint16_t)(r.y & 0xFFFF));
            acc.w += bf16_to_f32((uint16_t)(r.y >> 16));
        }
        if (a.out_f32) {
            *reinterpret_cast<float4 *>(reinterpret_cast<float *>(a.out) + o) = acc;
        } else {
            const u32 lo = (u32)f32_to_bf16_rne(acc.x) | ((u32)f32_to_bf16_rne(acc.y) << 16);
            const u32 hi = (u32)f32_to_bf16_rne(acc.z) | ((u32)f32_to_bf16_rne(acc.w) << 16);
            *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(a.out) + o) = make_uint2(lo, hi);
        }
    }
}

}  // namespace moeq
