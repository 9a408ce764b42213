// prefill.h -- the MoE layer for many tokens at once, on the matrix cores.
//
// With a prompt chunk of 2,048 tokens and top-10 of 512 experts each expert
// sees about 40 tokens, enough rows for the bf16 matrix instructions to pay
// (knivesysl "Prompt processing" notes; Strata SYCL port, "MoE prefill").
// A chunk runs as four launches on one stream:
//
//   route and group  top-k per token (one wave each), each pick claiming a
//            place in its expert slot's token list; the last workgroup to
//            finish turns the counts into pair offsets and a list of blocks
//            of up to 64 tokens of one slot (calls for one fixed expert:
//            pf_group_kernel, one workgroup per slot, instead)
//   gate/up  per (block, tile of 64 intermediate rows; 128 for the
//            256-wide and the scaled kernels below): g = Wg x, u = Wu x
//            on MFMA 16x16x32 bf16 with fp32 accumulation, then
//            h = silu(g) * u, stored as a bf16 hi + lo pair
//   down     y = Wd (h_hi + h_lo) into fp32 partials, one row per (token,
//            expert) pair: for K of 256..512 a persistent grid (one
//            workgroup per CU) shares out the 256-row passes of every block,
//            each block's h resident in LDS; otherwise per (block, tile of
//            512 hidden rows, 256 for six-bit codes)
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
// LDS, in a ring of stages, and read by all four waves.
//
// LDS banks (measured with the bank-conflict counter on the three staged
// layouts here): a 16-byte read is served 32 lanes at a time across 512 bytes
// of banks, so the 16 rows of one lane group and the 16 rows of the next must
// together cover 32 distinct 16-byte slots of a 512-byte window.  The
// swizzles below XOR a piece index with a row function whose bit 2 is zero:
// lane groups whose pieces differ in bit 2 then never meet, and within one
// lane group the function is one-to-one over the rows that share a window.
// (The resident-down, 256-wide and MX tiles count no conflicts this way; the
// 128-wide gate/up kernel still counts them on about half of its LDS cycles,
// unchanged by a swizzle that is conflict-free under every lane grouping that
// fits the other tiles' counts, so their source there is not its A reads.)
#pragma once

#include <type_traits>

#include "common.h"
#include "memops.h"
#include "mfma_unit.h"

namespace moeq {


// Row swizzles (see "LDS banks" above): 256-byte rows (two rows per 512-byte
// window; one-to-one over the 8 rows of each parity) and 1 KiB rows (one
// window per 32 pieces; one-to-one over 16 rows).
__host__ __device__ constexpr int pf_swz256(int r) { return ((r >> 1) & 3) | (r & 8); }
__host__ __device__ constexpr int pf_swz1k(int r) { return (r & 3) | ((r & 12) << 1); }

constexpr int PF_THREADS = 256;
constexpr int PF_MB = 64;                   // tokens per block (four 16-row sub-tiles)
constexpr int PF_KS = 128;                  // K per step
constexpr int PF_ROW = PF_KS * 2 + 16;      // bytes per staged activation row
constexpr int PF_STAGE = PF_MB * PF_ROW;    // bytes per staged plane
constexpr int PF_RG_GU = 1;                 // 16-row groups per wave: gate/up (each of gate and up)
// down: e2m1 takes four (measured: 2 -> 4 took 10 us off the 2,048-token
// layer); six-bit codes' larger units would spill registers with four
template <int FMT> constexpr int pf_rg_dn() { return Fmt<FMT>::SIX ? 2 : 4; }
constexpr int PF_PD = 2;                    // weight units in flight per row group (K steps ahead; three
                                            // measured 1-3 % slower: fewer rows open per CU)
constexpr int PF_MAX_K = 32;                // top-k limit of the layer

struct PfArgs {
    LayerArgs L;
    const uint16_t *x;        // bf16 [T][H] of the chunk
    int T;                    // tokens in the chunk
    int NS;                   // expert slots: E routed, +1 shared (slot E)
    int mode, fixed_e;
    int32_t *idx;             // [T][k] (route mode; written by pf_route_group_kernel)
    float *w;                 // [T][k]
    const float *logits;      // [T][E] router logits of the chunk (route mode)
    int32_t *rank;            // [T][k]: position of the token in its expert's list
    int32_t *cnt;             // [NS]
    int32_t *off;             // [NS + 1]: first pair of each slot
    int32_t *nblk;            // [1]
    int32_t *blk;             // [nblk_max]: slot << 16 | first token of the block
    int32_t *tok;             // [NS][T]: token ids of each slot (in claim order when routed)
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
// header words WS_PF_CLAIM + s: tokens claimed by slot s while the routing
// kernel groups them (zero at rest: the last workgroup resets them); above the
// decode kernels' per-group and per-slice counters
constexpr int WS_PF_CLAIM = 2048;
constexpr int PF_MAX_SLOTS = 1024 + 1;   // routed experts (the C ABI's limit) and the shared one
static_assert(WS_PF_CLAIM + PF_MAX_SLOTS <= (int)(WS_HEADER / 4), "claim words inside the header");

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

// Exclusive scan over the NT threads of a block (values in v, total returned;
// s_tmp holds NT / 64 ints).
template <int NT>
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
    total = 0;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
        if (i < wv) base += s_tmp[i];
        total += s_tmp[i];
    }
    __syncthreads();
    return base + x - v;
}

// The plan, built by the last workgroup of a grouping launch from the slots'
// counts (in LDS: s_cnt[s] for every slot): pair offsets and the block list,
// slot by slot in ascending order; then the arrival counter goes back to zero.
template <int NT>
__device__ inline void pf_build_plan(const PfArgs &a, const int *s_cnt, int *s_tmp, int tid) {
    const int NS = a.NS;
    const int per = (NS + NT - 1) / NT;
    const int s0 = tid * per;
    int c_sum = 0, b_sum = 0;
    for (int s = s0; s < s0 + per && s < NS; ++s) {
        const int c = s_cnt[s];
        c_sum += c;
        b_sum += (c + PF_MB - 1) / PF_MB;
    }
    int c_tot, b_tot;
    int c_base = pf_block_scan<NT>(c_sum, s_tmp, tid, c_tot);
    int b_base = pf_block_scan<NT>(b_sum, s_tmp, tid, b_tot);
    for (int s = s0; s < s0 + per && s < NS; ++s) {
        const int c = s_cnt[s];
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
    __shared__ int s_cnt[PF_MAX_SLOTS];
    for (int s = tid; s < a.NS; s += PF_THREADS) s_cnt[s] = pf_ld_relaxed(&a.cnt[s]);
    __syncthreads();
    pf_build_plan<PF_THREADS>(a, s_cnt, s_tmp, tid);
}

// Route and group in one launch (route mode): wave w of workgroup b routes
// token 16b + w (top-k with ties to the lower index, softmax over the picks),
// and each of its k picks claims the next place in its expert's token list
// with a device-scope atomic on that slot's header word.  The places depend
// on the order in which the claims arrive, so the lists and the pairs' ranks
// may differ from run to run; the outputs do not: every token's row is
// multiplied and combined the same way whatever its place in a block (the
// matrix instructions keep rows apart, and the combine follows rank order).
// The last workgroup to arrive moves the claims into cnt[] (the shared slot
// takes every token), resets the claim words and builds the plan.  Sixteen
// waves to a workgroup keep the arrivals on the one counter word few.
constexpr int PF_RG_THREADS = 1024;
template <int PER_LANE>
__global__ __launch_bounds__(PF_RG_THREADS) void pf_route_group_kernel(PfArgs a) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int T = a.T, k = a.L.k, E = a.L.E;
    __shared__ int s_tmp[PF_RG_THREADS / 64];
    __shared__ int s_last;
    int32_t *claim = reinterpret_cast<int32_t *>(a.hdr) + WS_PF_CLAIM;
    const int t = blockIdx.x * (PF_RG_THREADS / 64) + (tid >> 6);
    if (t < T) {   // uniform over the wave
        int e;
        float wt;
        route_one_token_wave<PER_LANE>(a.logits + (int64_t)t * E, E, k, lane, e, wt);
        if (lane < k) {
            a.idx[(int64_t)t * k + lane] = e;
            a.w[(int64_t)t * k + lane] = wt;
            // a token picks a slot at most once, so p < T while the claim words
            // start at zero; a place past the list (a workspace that was not
            // zeroed) is compared before any address is formed from it
            const int p = __hip_atomic_fetch_add(&claim[e], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (p < T) a.tok[(size_t)e * T + p] = t;
            a.rank[(int64_t)t * k + lane] = p < T ? p : 0;   // always a place inside the slot
        }
        if (lane == 0 && a.NS > E) a.tok[(size_t)E * T + t] = t;
    }
    __syncthreads();   // (with every load and store of the workgroup complete)
    if (tid == 0) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        const u32 prev = __hip_atomic_fetch_add(&a.hdr[WS_PF_ARRIVE], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (prev == gridDim.x - 1u) ? 1 : 0;
    }
    __syncthreads();
    if (!s_last) return;
    __shared__ int s_cnt[PF_MAX_SLOTS];
    for (int s = tid; s < a.NS; s += PF_RG_THREADS) {
        int c = (s == E) ? T : pf_ld_relaxed(&claim[s]);
        if (c < 0 || c > T) {   // claims past the list: reported, the count kept inside it
            pf_st_relaxed(reinterpret_cast<int32_t *>(&a.hdr[WS_ERR]), 1);
            c = c < 0 ? 0 : T;
        }
        s_cnt[s] = c;
        a.cnt[s] = c;
        pf_st_relaxed(&claim[s], 0);
    }
    __syncthreads();
    pf_build_plan<PF_RG_THREADS>(a, s_cnt, s_tmp, tid);
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
// 256 bytes (128 bf16); the 16-byte piece c of row r sits at c ^ pf_swz256(r),
// so the 32 rows-and-pieces that one half-wave reads for an MFMA fill a
// 512-byte bank window exactly.
template <int FMT, bool DOWN, int NSUB, int NWAVES, int RG>
__device__ inline void pf_gemm_main(const PfArgs &a, uint8_t *st0, uint8_t *st1, uint8_t *st2,
                                    const float *s_scale, const int *s_tok, int M,
                                    int p0, int K, int N, int n0, const uint8_t *const (&rc)[DOWN ? RG : 2 * RG],
                                    const uint8_t *const (&rs)[DOWN ? RG : 2 * RG]) {
    constexpr int NB = DOWN ? RG : 2 * RG;
    constexpr int NPL = DOWN ? 2 : 1;
    constexpr int PLANE = NSUB * 16 * 256;                  // bytes per plane of a stage
    constexpr int R = PF_PD + 1;                            // stages in the ring (separate LDS objects)
    static_assert(R == 3, "three stage objects");
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
        const int logical = (P & 15) ^ pf_swz256(row);
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
        else return st2;
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
    // prologue: steps 0 .. PD-1 in flight
    issue_stage(I0{}, 0);
    load_w(wq[0], 0);
    issue_stage(I1{}, 1);
    load_w(wq[1], 1);

    // step it uses stage and weight slot it % 3 and refills slot (it + 2) % 3
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
            const int piece = ((lg * 4 + s) ^ pf_swz256(lr)) * 16;
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
    }
    if (it < nK) step(I0{}, it);
    if (it + 1 < nK) step(I1{}, it + 1);
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
        case 1: pf_gemm_main<FMT, DOWN, 1, NWAVES, RG>(a, pf_st0, pf_st1, pf_st2, s_scale, s_tok, M, p0, K, N, n0, rc, rs); break;
        case 2: pf_gemm_main<FMT, DOWN, 2, NWAVES, RG>(a, pf_st0, pf_st1, pf_st2, s_scale, s_tok, M, p0, K, N, n0, rc, rs); break;
        case 3: pf_gemm_main<FMT, DOWN, 3, NWAVES, RG>(a, pf_st0, pf_st1, pf_st2, s_scale, s_tok, M, p0, K, N, n0, rc, rs); break;
        default: pf_gemm_main<FMT, DOWN, 4, NWAVES, RG>(a, pf_st0, pf_st1, pf_st2, s_scale, s_tok, M, p0, K, N, n0, rc, rs); break;
    }
}

// Gate | up with bf16 activations on 256-wide K steps (H a multiple of 256;
// used for the UE8M0 formats): the shape of the scaled kernel below, for the
// bf16 matrix instructions.  A
// workgroup of eight waves takes (block of up to 64 tokens, tile of 128
// intermediate rows); each wave owns 16 gate and the same 16 up rows.  Per K
// step a lane loads two consecutive units of each of its rows, 8s + 2h and
// 8s + 2h + 1 (the four lane groups read 64 contiguous code bytes of a row,
// or 96 for six-bit codes), decodes them as pf_unit_to_b does, and MFMA
// (t, q) of the step takes weights 8q .. 8q+7 of unit 8s + 2h + t in lane
// group h: K offsets 64h + 32t + 8q.  The activations are read with the same
// mapping from a 64 x 512-byte stage (piece 8h + 4t + q of the row, XORed
// with pf_swz512 of the row).  Two K steps in flight, three stages of 32 KiB,
// one workgroup per CU.
constexpr int PF_G2_KS = 256;
constexpr int PF_G2_ROW = PF_G2_KS * 2;        // bytes per staged bf16 row
constexpr int PF_G2_NW = 8;
constexpr int PF_G2_PD = 2;
// 512-byte rows: one bank window per row; one-to-one over 16 rows, bit 3 clear
__host__ __device__ constexpr int pf_swz512(int r) { return (r & 7) | ((r & 8) << 1); }

template <int FMT, int NSUB>
__device__ inline void pf_gu256_main(const PfArgs &a, uint8_t *st0, uint8_t *st1, uint8_t *st2, const float *s_scale,
                                     const int *s_tok, int M, int p0, int Is, int n0,
                                     const uint8_t *const (&rc)[2], const uint8_t *const (&rs)[2]) {
    constexpr int NW = PF_G2_NW, NB = 2, PD = PF_G2_PD, R = PD + 1;
    static_assert(R == 3, "three stage objects");
    constexpr int NDMA = NSUB * 16 * PF_G2_ROW / 1024;  // 1 KiB copies per stage
    static_assert(NDMA % NW == 0, "copies per wave");
    constexpr int DPW = NDMA / NW;
    constexpr int PER_GROUP = DPW + NB * 2 * PfUnitLoads<FMT>::n;
    constexpr bool WLO = pf_split_w<FMT>();
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int lg = lane >> 4, lr = lane & 15;
    const int H = a.L.H;
    const int nK = H / PF_G2_KS;

    const __amdgpu_buffer_rsrc_t src = rsrc_of(a.x, (uint64_t)a.T * H * 2);
    u32 row_off[DPW], col_k[DPW];
    int dst_off[DPW];
#pragma unroll
    for (int q = 0; q < DPW; ++q) {
        const int g = q * NW + wv;                      // copy index in the stage
        const int P = g * 64 + lane;                    // 16-byte position in the stage
        const int row = P >> 5;
        const int logical = (P & 31) ^ pf_swz512(row);
        row_off[q] = (u32)s_tok[min(row, M - 1)] * (u32)H * 2u;
        col_k[q] = (u32)logical * 16u;
        dst_off[q] = g * 1024;
    }
    auto stage = [&](auto sc) -> uint8_t * {
        constexpr int S = decltype(sc)::value;
        if constexpr (S == 0) return st0;
        else if constexpr (S == 1) return st1;
        else return st2;
    };
    Unit<FMT> wq[R][NB][2];
    auto issue = [&](auto sc, int j) {
        constexpr int S = decltype(sc)::value;
        uint8_t *st = stage(sc);
        const int jj = min(j, nK - 1);                  // past the end: the last step again, unused
        const u32 kb = (u32)jj * PF_G2_ROW;
#pragma unroll
        for (int q = 0; q < DPW; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_void_t *)(st + dst_off[q]), 16, row_off[q] + kb + col_k[q],
                                                     0, 0, 0);
        const int u0 = jj * 8 + 2 * lg;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            load_unit<FMT>(wq[S][b][0], rc[b], rs[b], u0);
            load_unit<FMT>(wq[S][b][1], rc[b], rs[b], u0 + 1);
        }
    };

    f32x4_t acc[NB][NSUB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int m = 0; m < NSUB; ++m) acc[b][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    issue(I0{}, 0);
    issue(I1{}, 1);

    auto step = [&](auto dc, int it) {
        constexpr int d = decltype(dc)::value;
        constexpr int dn = (d + PD) % R;
        pf_wait_vm<(PD - 1) * PER_GROUP>();             // this wave's step-it loads have landed
        pf_barrier();                                   // ... and every wave's; stage (it-1) % R is free
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            pf_pin_unit<FMT>(wq[d][b][0]);
            pf_pin_unit<FMT>(wq[d][b][1]);
        }
        issue(std::integral_constant<int, dn>{}, it + PD);
        asm volatile("" ::: "memory");
        const uint8_t *st = stage(dc);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            bf16x8_t bw[NB][4], bwl[NB][4];
#pragma unroll
            for (int b = 0; b < NB; ++b) pf_unit_to_b<FMT>(wq[d][b][t], s_scale, bw[b], bwl[b]);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int piece = 8 * lg + 4 * t + q;
                bf16x8_t ah[NSUB];
#pragma unroll
                for (int m = 0; m < NSUB; ++m) {
                    const int row = 16 * m + lr;
                    ah[m] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t *>(
                                                              st + row * PF_G2_ROW + ((piece ^ pf_swz512(row)) << 4)));
                }
#pragma unroll
                for (int m = 0; m < NSUB; ++m)
#pragma unroll
                    for (int b = 0; b < NB; ++b) {
                        acc[b][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[m], bw[b][q], acc[b][m], 0, 0, 0);
                        if (WLO) acc[b][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[m], bwl[b][q], acc[b][m], 0, 0, 0);
                    }
            }
        }
    };
    int it = 0;
    for (; it + R <= nK; it += R) {
        step(I0{}, it);
        step(I1{}, it + 1);
        step(I2{}, it + 2);
    }
    if (it < nK) step(I0{}, it);
    if (it + 1 < nK) step(I1{}, it + 1);
    pf_wait_vm<0>();    // the copies issued past the end land before the workgroup's LDS is reused

    // epilogue: lane holds tokens 16m + 4 lg + i, weight row n0 + 16 wv + lr
    const int nn = n0 + wv * 16 + lr;
    if (nn >= Is) return;
#pragma unroll
    for (int m = 0; m < NSUB; ++m) {
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

// One workgroup (eight waves) per (block of up to 64 tokens, tile of 128
// intermediate rows); the tiles of one block share an XCD.
template <int FMT>
__global__ __launch_bounds__(512, 1) void pf_gu256_kernel(PfArgs a, int NT) {
    constexpr int STAGE_BYTES = PF_MB * PF_G2_ROW;
    __shared__ __attribute__((aligned(1024))) uint8_t g2_st0[STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t g2_st1[STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t g2_st2[STAGE_BYTES];
    __shared__ float s_scale[LUT_SCALE];
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
    const int n0 = nt * PF_G2_NW * 16;
    if (n0 >= Is) return;
    const int M = min(PF_MB, a.cnt[slot] - m0);
    const int nsub = (M + 15) >> 4;
    const int p0 = a.off[slot] + m0;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int lr = lane & 15;
    if (Fmt<FMT>::SCALE == SC_E4M3) {   // the other scales are converted arithmetically
        Luts Lt;
        Lt.pair = nullptr;
        Lt.scale = s_scale;
        build_luts<FMT>(Lt, tid, 64 * PF_G2_NW, false);
    }
    if (tid < PF_MB) s_tok[tid] = a.tok[(size_t)slot * a.T + m0 + min(tid, M - 1)];

    using F = Fmt<FMT>;
    const int64_t crb = F::code_row_bytes(H), srb = F::scale_row_bytes(H);
    const uint8_t *wc = shared ? a.L.sh13c : a.L.w13c + (size_t)slot * 2 * Is * crb;
    const uint8_t *ws = shared ? a.L.sh13s : a.L.w13s + (size_t)slot * 2 * Is * srb;
    const int n = min(n0 + wv * 16 + lr, Is - 1);     // rows past Is: a valid row, result dropped
    const uint8_t *const rc[2] = {wc + (size_t)n * crb, wc + (size_t)(Is + n) * crb};
    const uint8_t *const rs[2] = {ws + (size_t)n * srb, ws + (size_t)(Is + n) * srb};
    __syncthreads();   // s_tok, scale table
    switch (nsub) {
        case 1: pf_gu256_main<FMT, 1>(a, g2_st0, g2_st1, g2_st2, s_scale, s_tok, M, p0, Is, n0, rc, rs); break;
        case 2: pf_gu256_main<FMT, 2>(a, g2_st0, g2_st1, g2_st2, s_scale, s_tok, M, p0, Is, n0, rc, rs); break;
        case 3: pf_gu256_main<FMT, 3>(a, g2_st0, g2_st1, g2_st2, s_scale, s_tok, M, p0, Is, n0, rc, rs); break;
        default: pf_gu256_main<FMT, 4>(a, g2_st0, g2_st1, g2_st2, s_scale, s_tok, M, p0, Is, n0, rc, rs); break;
    }
}

// Down projection with the block's h resident in LDS.  y = Wd (h_hi + h_lo)
// has a short K (the intermediate width, 512 here), so a workgroup per (block,
// tile of rows) would spend most of its life filling its pipeline.  Instead
// one workgroup of eight waves takes a run of passes of a block: it copies the
// block's h_hi and h_lo rows into LDS once (64 rows x 1 KiB per plane), and
// every wave then streams its weight rows for the run's outputs, 32 rows (two
// 16-row groups) per pass, with PD K steps of weight units in flight in registers and no
// barrier after the copy -- the weights are private to the wave.  Row r of a
// plane is 1 KiB; its 16-byte chunk c sits at c ^ pf_swz1k(r) (inside its
// 32-chunk window), so a half-wave's 32 reads fall on distinct banks.
//
// Each pass ends with its y stores.  On this part vmcnt counts stores as well
// as loads, and a store may complete before older loads, so the only safe
// wait for a load group is "at most (younger loads) outstanding", which also
// waits for every store issued since.  The pass's last step therefore waits
// for the next step's group before it issues the stores, that next step
// skips its wait, and the stores have its whole compute time to complete
// before the step after it waits again.
constexpr int PF_DR_KMAX = 512;
constexpr int PF_DR_RG = 2;                 // 16-row groups per wave per pass
constexpr int PF_DR_PLANE = PF_MB * PF_DR_KMAX * 2;
// K steps in flight: 4 when a pass has 4 K steps (K = 512), else 2 (K = 256, 384)

template <int FMT, int NSUB, int PD>
__device__ inline void pf_down_res_main(const PfArgs &a, uint8_t *s_h, const float *s_scale, int M, int p0, int K,
                                        const uint8_t *wc, const uint8_t *ws, int ps_lo, int ps_hi) {
    constexpr int NWAVES = 8, RG = PF_DR_RG, R = PD + 1;
    constexpr int PER_GROUP = RG * PfUnitLoads<FMT>::n;
    constexpr int T0 = (PD - 1) * PER_GROUP;            // loads younger than a step's group
    constexpr bool WLO = pf_split_w<FMT>();
    constexpr int CP = 2 * 16 * NSUB / NWAVES;          // 1 KiB row copies per wave (both planes)
    static_assert((2 * 16 * NSUB) % NWAVES == 0, "copies per wave");
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int lg = lane >> 4, lr = lane & 15;
    const int H = a.L.H;
    const int nK = K / PF_KS;                           // K steps per pass (>= PD)
    constexpr int ROWS = NWAVES * RG * 16;              // rows per pass
    const int nstep = (ps_hi - ps_lo) * nK;             // passes ps_lo .. ps_hi - 1 of the block
    using F = Fmt<FMT>;
    const int64_t crb = F::code_row_bytes(K), srb = F::scale_row_bytes(K);

    // the block's h rows into LDS: copy q of this wave is row (q * 8 + wv) of
    // the two planes; lane = the row's 16-byte position, holding chunk lane ^ pf_swz1k(row)
    {
        const uint64_t bytes = (uint64_t)a.off[a.NS] * a.Imax * 2;
        const __amdgpu_buffer_rsrc_t src[2] = {rsrc_of(a.h_hi, bytes), rsrc_of(a.h_lo, bytes)};
#pragma unroll
        for (int q = 0; q < CP; ++q) {
            const int g = q * NWAVES + wv;              // 0 .. 32 NSUB - 1
            constexpr int HALF = CP / 2;                // copies q < HALF are h_hi rows (g < 16 NSUB)
            const int pl = q < HALF ? 0 : 1, row = g - pl * 16 * NSUB;
            const int c = lane ^ pf_swz1k(row);
            const u32 voff = c * 8 < K ? ((u32)(p0 + min(row, M - 1)) * (u32)a.Imax + (u32)c * 8u) * 2u : 0x7FFFFFF0u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(src[pl], (lds_void_t *)(s_h + pl * PF_DR_PLANE + row * 1024), 16,
                                                     voff, 0, 0, 0);
        }
    }
    asm volatile("" ::: "memory");     // the copies are issued before the weight loads below

    // weight units of flattened step f = pass * nK + j: unit 4 j + lg of rows
    // pass * ROWS + wv * 32 + 16 g + lr (clamped into the matrix; results dropped)
    Unit<FMT> wq[R][RG];
    auto load_w = [&](Unit<FMT> (&U)[RG], int f) {
        const int ff = min(f, nstep - 1);
        const int ps = ps_lo + ff / nK, j = ff - (ps - ps_lo) * nK;
#pragma unroll
        for (int g = 0; g < RG; ++g) {
            const int n = min(ps * ROWS + wv * 16 * RG + 16 * g + lr, H - 1);
            load_unit<FMT>(U[g], wc + (size_t)n * crb, ws + (size_t)n * srb, 4 * j + lg);
        }
    };
    f32x4_t acc[RG][NSUB];
#pragma unroll
    for (int g = 0; g < RG; ++g)
#pragma unroll
        for (int m = 0; m < NSUB; ++m) acc[g][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    [&]<int... I>(std::integer_sequence<int, I...>) { (load_w(wq[I], I), ...); }(std::make_integer_sequence<int, PD>{});
    pf_wait_vm<PD * PER_GROUP>();                       // this wave's h copies have landed
    pf_barrier();                                       // ... and every wave's (weights stay in flight)

    auto step = [&](auto dc, int f) {
        constexpr int d = decltype(dc)::value;
        constexpr int dn = (d + PD) % R;
        const int ps = ps_lo + f / nK, j = f - (ps - ps_lo) * nK;
        // step f's units have landed (the first step of a pass: waited for
        // before the previous pass's stores)
        if (!(ps > ps_lo && j == 0)) pf_wait_vm<T0>();
#pragma unroll
        for (int g = 0; g < RG; ++g) pf_pin_unit<FMT>(wq[d][g]);
        bf16x8_t bw[RG][4], bwl[RG][4];
#pragma unroll
        for (int g = 0; g < RG; ++g) pf_unit_to_b<FMT>(wq[d][g], s_scale, bw[g], bwl[g]);
        load_w(wq[dn], f + PD);
        asm volatile("" ::: "memory");                  // the stores below stay after these loads
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int c = 16 * j + 4 * lg + s;          // chunk: K 8c .. 8c+7
            bf16x8_t ah[NSUB], al[NSUB];
#pragma unroll
            for (int m = 0; m < NSUB; ++m) {
                const int row = 16 * m + lr;
                const uint8_t *ap = s_h + row * 1024 + ((c ^ pf_swz1k(row)) << 4);
                ah[m] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t *>(ap));
                al[m] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t *>(ap + PF_DR_PLANE));
            }
#pragma unroll
            for (int m = 0; m < NSUB; ++m)
#pragma unroll
                for (int g = 0; g < RG; ++g) {
                    acc[g][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[m], bw[g][s], acc[g][m], 0, 0, 0);
                    acc[g][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[m], bw[g][s], acc[g][m], 0, 0, 0);
                    if (WLO) {
                        acc[g][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[m], bwl[g][s], acc[g][m], 0, 0, 0);
                        acc[g][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[m], bwl[g][s], acc[g][m], 0, 0, 0);
                    }
                }
        }
        if (j == nK - 1) {
            pf_wait_vm<T0>();                           // step f + 1's units, before any store
            // the pass's stores: lane holds tokens 16m + 4 lg + i of row n
#pragma unroll
            for (int g = 0; g < RG; ++g) {
                const int n = ps * ROWS + wv * 16 * RG + 16 * g + lr;
#pragma unroll
                for (int m = 0; m < NSUB; ++m) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = 16 * m + 4 * lg + i;
                        if (n < H && t < M) a.y[(size_t)(p0 + t) * H + n] = acc[g][m][i];
                    }
                    acc[g][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                }
            }
        }
    };
    int f = 0;
    for (; f + R <= nstep; f += R)
        [&]<int... I>(std::integer_sequence<int, I...>) {
            (step(std::integral_constant<int, I>{}, f + I), ...);
        }(std::make_integer_sequence<int, R>{});
    [&]<int... I>(std::integer_sequence<int, I...>) {
        ((f + I < nstep ? step(std::integral_constant<int, I>{}, f + I) : void()), ...);
    }(std::make_integer_sequence<int, R - 1>{});
    pf_wait_vm<0>();    // the loads issued past the end land before the wave exits
}

// Down with the h rows resident: a persistent grid of eight-wave workgroups
// (one per CU) shares out the passes of every block (ROWS output rows each)
// evenly, in block order, so no CU idles while the last blocks run.  A
// workgroup whose passes span several blocks copies each block's h rows into
// LDS when it reaches it.  Every pass of a block computes all K for its rows,
// so the results do not depend on how the passes are shared out.
template <int FMT>
__global__ __launch_bounds__(512, 1) void pf_down_res_kernel(PfArgs a) {
    __shared__ __attribute__((aligned(1024))) uint8_t s_h[2 * PF_DR_PLANE];
    __shared__ float s_scale[LUT_SCALE];
    const int E = a.L.E, H = a.L.H;
    constexpr int ROWS = 8 * PF_DR_RG * 16;
    const int npass = (H + ROWS - 1) / ROWS;
    const int64_t total = (int64_t)a.nblk[0] * npass;
    const int q0 = (int)(total * blockIdx.x / gridDim.x), q1 = (int)(total * (blockIdx.x + 1) / gridDim.x);
    if (q0 >= q1) return;
    if (Fmt<FMT>::SCALE == SC_E4M3) {   // the other scales are converted arithmetically
        Luts Lt;
        Lt.pair = nullptr;
        Lt.scale = s_scale;
        build_luts<FMT>(Lt, threadIdx.x, 512, false);
        __syncthreads();
    }
    using F = Fmt<FMT>;
    for (int q = q0; q < q1;) {
        const int b = q / npass, ps_lo = q - b * npass;
        const int ps_hi = min(npass, ps_lo + (q1 - q));
        const int packed = a.blk[b];
        const int slot = packed >> 16, m0 = packed & 0xFFFF;
        const bool shared = slot == E;
        const int K = shared ? a.L.Ish : a.L.I;
        const int M = min(PF_MB, a.cnt[slot] - m0);
        const int nsub = (M + 15) >> 4;
        const int p0 = a.off[slot] + m0;
        const int64_t crb = F::code_row_bytes(K), srb = F::scale_row_bytes(K);
        const uint8_t *wc = shared ? a.L.sh2c : a.L.w2c + (size_t)slot * H * crb;
        const uint8_t *ws = shared ? a.L.sh2s : a.L.w2s + (size_t)slot * H * srb;
        if (q != q0) __syncthreads();   // every wave is done with the previous block's h rows
        // two K steps of weight units in flight (I = 512: 0.423 ms for the step
        // against 0.429 with four; fewer rows' loads open per CU)
        switch (nsub) {
            case 1: pf_down_res_main<FMT, 1, 2>(a, s_h, s_scale, M, p0, K, wc, ws, ps_lo, ps_hi); break;
            case 2: pf_down_res_main<FMT, 2, 2>(a, s_h, s_scale, M, p0, K, wc, ws, ps_lo, ps_hi); break;
            case 3: pf_down_res_main<FMT, 3, 2>(a, s_h, s_scale, M, p0, K, wc, ws, ps_lo, ps_hi); break;
            default: pf_down_res_main<FMT, 4, 2>(a, s_h, s_scale, M, p0, K, wc, ws, ps_lo, ps_hi); break;
        }
        q += ps_hi - ps_lo;
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
//
// A K step is 256 wide (eight 32-weight units), two instructions.  Each lane
// loads two consecutive units of its row, 8s + 2h and 8s + 2h + 1 (so the four
// lane groups read 128 contiguous bytes of the row for e2m1), and instruction
// t of the step takes unit 8s + 2h + t in lane group h.  A dot product does
// not care in which order its terms are summed, so the instruction's K block b
// simply is unit 8s + 2b + t: lane group g then takes, from the staged codes,
// the half g%2 of units 8s + 2(g/2) + t and 8s + 4 + 2(g/2) + t, and the scale
// of activation block 8s + 2g + t.
//
// The pipeline is the bf16 path's (pf_gemm_main) with two steps in flight:
// the 64 x 256 byte code tile of a K step is copied into an LDS stage by
// buffer-load-to-LDS, two steps ahead, together with each lane's weight units and its two activation scale
// bytes per 16-token sub-tile, so one vmcnt wait per step covers all of them.
// Stage rows are 256 bytes; the 16-byte piece c of row r sits at c ^ (r & 15),
// so the 16 rows a quarter-wave reads fall on distinct banks.  H must be a
// multiple of 256 (every unit of every step is then inside the row).
typedef __attribute__((ext_vector_type(8))) int v8i_t;

constexpr int PF_MX_KS = 256;                         // K per step = bytes per staged e4m3 row
constexpr int PF_MX_PD = 2;                           // K steps in flight

// Two consecutive weight units of a row (codes) and their scale byte(s).
template <int FMT> struct MxPair {
    static constexpr int ND = Fmt<FMT>::SIX ? 12 : 8;
    u32 c[ND];
    u32 s;
};

template <int FMT>
__device__ inline void mx_load_pair(MxPair<FMT> &P, const uint8_t *codes, const uint8_t *scales, int u0) {
    const uint8_t *p = codes + (int64_t)u0 * Fmt<FMT>::UNIT_CODE_BYTES;
#pragma unroll
    for (int q = 0; q < MxPair<FMT>::ND / 4; ++q) {
        const uint4 v = ldg16(p + 16 * q);
        P.c[4 * q] = v.x; P.c[4 * q + 1] = v.y; P.c[4 * q + 2] = v.z; P.c[4 * q + 3] = v.w;
    }
    if constexpr (Fmt<FMT>::BLOCK == 32) P.s = *reinterpret_cast<const uint16_t *>(scales + u0);   // u0 even
    else P.s = scales[u0 / (Fmt<FMT>::BLOCK / 32)];                 // both units in one block
}

// B operand and scale byte of unit t (0, 1) of the pair
template <int FMT>
__device__ inline v8i_t mx_b(const MxPair<FMT> &P, int t) {
    v8i_t v = {0, 0, 0, 0, 0, 0, 0, 0};
    constexpr int W = Fmt<FMT>::SIX ? 6 : 4;
#pragma unroll
    for (int i = 0; i < W; ++i) v[i] = (int)P.c[W * t + i];
    return v;
}
template <int FMT>
__device__ inline int mx_bs(const MxPair<FMT> &P, int t) {
    return Fmt<FMT>::BLOCK == 32 ? (int)((P.s >> (8 * t)) & 0xFF) : (int)(P.s & 0xFF);
}

// An empty asm that "rewrites" the registers: placed after the step's vmcnt
// wait, it keeps the compiler from hoisting their uses above that wait (its
// own waitcnt pass would then also wait for younger loads).
template <int FMT>
__device__ inline void mx_pin(MxPair<FMT> &P) {
#pragma unroll
    for (int i = 0; i < MxPair<FMT>::ND; ++i) asm volatile("" : "+v"(P.c[i]));
    asm volatile("" : "+v"(P.s));
}

template <int FMT, int NSUB>
__device__ inline void pf_mx_main(const PfArgs &a, uint8_t *st0, uint8_t *st1, uint8_t *st2,
                                  const int *s_tok, int M, int p0, int Is, int n0, const uint8_t *const (&rc)[2],
                                  const uint8_t *const (&rs)[2]) {
    constexpr int NWAVES = 4, NB = 2;
    constexpr int BFMT = Fmt<FMT>::SIX ? 2 : 4;        // fp6 e2m3 or fp4 e2m1 operand
    constexpr int PD = PF_MX_PD;
    constexpr int R = PD + 1;
    static_assert(R == 3, "three stage objects");
    constexpr int NDMA = NSUB * 16 * PF_MX_KS / 1024;  // 1 KiB copies per stage (4 per sub-tile)
    constexpr int DPW = NDMA / NWAVES;                 // = NSUB
    constexpr int PER_GROUP = DPW + NB * (MxPair<FMT>::ND / 4 + 1) + NSUB;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int lg = lane >> 4, lr = lane & 15;
    const int H = a.L.H, HB = H / 32;
    const int nK = H / PF_MX_KS;

    const __amdgpu_buffer_rsrc_t src = rsrc_of(a.xq, (uint64_t)a.T * H);
    u32 row_off[DPW], col_k[DPW];
    int dst_off[DPW];
#pragma unroll
    for (int q = 0; q < DPW; ++q) {
        const int g = q * NWAVES + wv;                 // copy index in the stage
        const int P = g * 64 + lane;                   // 16-byte position in the stage
        const int row = P >> 4;
        const int logical = (P & 15) ^ (row & 15);
        row_off[q] = (u32)s_tok[min(row, M - 1)] * (u32)H;
        col_k[q] = (u32)logical * 16u;
        dst_off[q] = g * 1024;
    }
    // this lane's activation scale rows (one per sub-tile)
    const uint8_t *srow[NSUB];
#pragma unroll
    for (int m = 0; m < NSUB; ++m) srow[m] = a.xs + (size_t)s_tok[min(16 * m + lr, M - 1)] * HB;

    auto stage = [&](auto sc) -> uint8_t * {
        constexpr int S = decltype(sc)::value;
        if constexpr (S == 0) return st0;
        else if constexpr (S == 1) return st1;
        else return st2;
    };
    MxPair<FMT> wq[R][NB];
    u32 sq[R][NSUB];
    // the loads of K step j (clamped to the last step past the end: no branch,
    // results unused): activation codes into stage sc, weight units and scale
    // bytes into register slot sc
    auto issue = [&](auto sc, int j) {
        constexpr int S = decltype(sc)::value;
        uint8_t *st = stage(sc);
        const int jj = min(j, nK - 1);
        const u32 kb = (u32)jj * PF_MX_KS;
#pragma unroll
        for (int q = 0; q < DPW; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_void_t *)(st + dst_off[q]), 16, row_off[q] + kb + col_k[q],
                                                     0, 0, 0);
        const int u0 = jj * 8 + 2 * lg;
#pragma unroll
        for (int b = 0; b < NB; ++b) mx_load_pair<FMT>(wq[S][b], rc[b], rs[b], u0);
#pragma unroll
        for (int m = 0; m < NSUB; ++m) sq[S][m] = *reinterpret_cast<const uint16_t *>(srow[m] + u0);
    };

    f32x4_t acc[NB][NSUB];
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int m = 0; m < NSUB; ++m) acc[j][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    issue(I0{}, 0);
    issue(I1{}, 1);

    auto step = [&](auto dc, int it) {
        constexpr int d = decltype(dc)::value;
        constexpr int dn = (d + PD) % R;
        pf_wait_vm<(PD - 1) * PER_GROUP>();          // this wave's step-it loads have landed
        pf_barrier();                                   // ... and every wave's; stage (it-1) % R is free
#pragma unroll
        for (int b = 0; b < NB; ++b) mx_pin<FMT>(wq[d][b]);
#pragma unroll
        for (int m = 0; m < NSUB; ++m) asm volatile("" : "+v"(sq[d][m]));
        issue(std::integral_constant<int, dn>{}, it + PD);
        const MxPair<FMT> (&w)[NB] = wq[d];
        const u32 (&sa)[NSUB] = sq[d];
        const uint8_t *st = stage(dc);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            // pieces 4(g/2) + 2t + g%2 and 8 + the same, of rows 16m + lr
            const int q0 = 4 * (lg >> 1) + 2 * t + (lg & 1);
#pragma unroll
            for (int m = 0; m < NSUB; ++m) {
                const int row = 16 * m + lr;
                const u32x4_t p0v = *reinterpret_cast<const u32x4_t *>(st + row * PF_MX_KS + ((q0 ^ (row & 15)) << 4));
                const u32x4_t p1v =
                    *reinterpret_cast<const u32x4_t *>(st + row * PF_MX_KS + (((8 + q0) ^ (row & 15)) << 4));
                const v8i_t av = {(int)p0v[0], (int)p0v[1], (int)p0v[2], (int)p0v[3],
                                  (int)p1v[0], (int)p1v[1], (int)p1v[2], (int)p1v[3]};
                const int sam = (int)((sa[m] >> (8 * t)) & 0xFF);
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    acc[b][m] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, mx_b<FMT>(w[b], t), acc[b][m], 0,
                                                                                 BFMT, 0, sam, 0, mx_bs<FMT>(w[b], t));
            }
        }
    };
    int it = 0;
    for (; it + R <= nK; it += R) {
        step(I0{}, it);
        step(I1{}, it + 1);
        step(I2{}, it + 2);
    }
    if (it < nK) step(I0{}, it);
    if (it + 1 < nK) step(I1{}, it + 1);
    pf_wait_vm<0>();    // the copies issued past the end land before the workgroup's LDS is reused

    // epilogue: lane holds tokens 16m + 4 lg + i, weight row n0 + 16 wv + lr
    const int nn = n0 + wv * 16 + lr;
    if (nn >= Is) return;
#pragma unroll
    for (int m = 0; m < NSUB; ++m) {
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

// One workgroup per (block of up to 64 tokens, tile of 64 intermediate rows):
// four waves, each with 16 rows of gate and the same 16 rows of up.
template <int FMT>
__global__ __launch_bounds__(256, 2) void pf_gateup_mx_kernel(PfArgs a, int NT) {
    static_assert(Fmt<FMT>::SCALE == SC_UE8M0, "MX weight formats only");
    constexpr int STAGE_BYTES = 4 * 16 * PF_MX_KS;
    __shared__ __attribute__((aligned(1024))) uint8_t mx_st0[STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t mx_st1[STAGE_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t mx_st2[STAGE_BYTES];
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
    const int nsub = (M + 15) >> 4;
    const int p0 = a.off[slot] + m0;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int lr = lane & 15;
    if (tid < PF_MB) s_tok[tid] = a.tok[(size_t)slot * a.T + m0 + min(tid, M - 1)];

    using F = Fmt<FMT>;
    const int64_t crb = F::code_row_bytes(H), srb = F::scale_row_bytes(H);
    const uint8_t *wc = shared ? a.L.sh13c : a.L.w13c + (size_t)slot * 2 * Is * crb;
    const uint8_t *ws = shared ? a.L.sh13s : a.L.w13s + (size_t)slot * 2 * Is * srb;
    const int n = min(n0 + wv * 16 + lr, Is - 1);     // rows past Is: a valid row, result dropped
    const uint8_t *const rc[2] = {wc + (size_t)n * crb, wc + (size_t)(Is + n) * crb};
    const uint8_t *const rs[2] = {ws + (size_t)n * srb, ws + (size_t)(Is + n) * srb};
    __syncthreads();   // s_tok
    switch (nsub) {
        case 1: pf_mx_main<FMT, 1>(a, mx_st0, mx_st1, mx_st2, s_tok, M, p0, Is, n0, rc, rs); break;
        case 2: pf_mx_main<FMT, 2>(a, mx_st0, mx_st1, mx_st2, s_tok, M, p0, Is, n0, rc, rs); break;
        case 3: pf_mx_main<FMT, 3>(a, mx_st0, mx_st1, mx_st2, s_tok, M, p0, Is, n0, rc, rs); break;
        default: pf_mx_main<FMT, 4>(a, mx_st0, mx_st1, mx_st2, s_tok, M, p0, Is, n0, rc, rs); break;
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
