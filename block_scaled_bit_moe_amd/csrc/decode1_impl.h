// decode1_impl.h -- the MoE layer for ONE token in one launch, shaped for
// latency (the decode step of nextsycl README, "What it does"; Strata
// docs/INTEL.md, "The engine itself on Intel": router_top10, shared_expert).
//
// With one token every selected expert serves exactly one row, so the work is
// static once the token is routed.  One workgroup of 16 waves on each of 7/8
// of the CUs (a burst of loads streams at the rate of the waves issuing it, so
// a CU needs many waves, not many loads per wave; and the fewer workgroups the
// h exchange waits for, the sooner it ends):
//   gate | up : the layer's P = k*I + Ish (gate row, up row) pairs, routed
//               experts in rank order then the shared expert, are split into
//               G equal ranges with even bounds; workgroup w computes range w
//               (it may straddle two experts);
//   down      : workgroup w computes RW consecutive output rows for EVERY
//               selected expert and combines them itself, in rank order, so no
//               partial sums leave the CU.
// Each workgroup routes the token itself (by ranks: every key compared with
// the others in parallel, no serial selection rounds), then issues all of its
// gate/up loads at once (into registers).  Its down rows are issued right after it
// has published its h and started reading everyone's: h is on the critical
// path, the down rows are not needed before all of h is in, and requests
// queue in issue order.  Every load is issued unconditionally (idle slots
// re-load a row the workgroup loads anyway), so the compiler counts
// outstanding loads exactly and waits only for the ones it needs.
//
//
// The down rows need every expert's h.  The gate and up rows of a pair sit in
// two slots of the same lane group, so that group's first lane has both dots
// and publishes h of the pair at once, as a 64-bit word (call tag << 32 |
// fp32 bits) with a device-coherent store: no barrier and no wait (every word
// carries its own tag, so no ordering between words is needed).  Then
// all 16 waves fetch every expert group's words, keep the payload of those
// whose tag is current (into LDS, compact and swizzled) and fetch again the
// groups that had a stale word, until all are in.  The first fetch uses
// ordinary loads, so the 32 workgroups of an XCD share one copy through its
// L2; later fetches bypass the L2.  The tag is the workspace's call counter +
// 1: every workgroup reads the counter on entry and raises it to counter + 1
// on exit.  That is safe because every workgroup publishes h and none leaves
// before all h is published, so none can finish before all have read the
// counter; and it stays correct when the launch is replayed from a captured
// graph.
#pragma once

#include <algorithm>

#include "kernels.h"
#include "rowdot.h"
#include "memops.h"

namespace moeq {

__device__ inline u32 d1_ld_relaxed(const u32 *p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ inline void d1_st_relaxed(u32 *p, u32 v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

// OR over the 64 lanes, returned uniform (same DPP stages as wave_max_u32)
__device__ inline u32 wave_or_u32(u32 v) {
    v |= dpp_mov_u32<0xB1>(v);
    v |= dpp_mov_u32<0x4E>(v);
    v |= dpp_mov_u32<0x141>(v);
    v |= dpp_mov_u32<0x140>(v);
    return (u32)__builtin_amdgcn_readlane((int)v, 0) | (u32)__builtin_amdgcn_readlane((int)v, 16) |
           (u32)__builtin_amdgcn_readlane((int)v, 32) | (u32)__builtin_amdgcn_readlane((int)v, 48);
}

constexpr int D1_NW = 16;                  // waves per workgroup
constexpr int D1_THREADS = 64 * D1_NW;
constexpr int D1_MAX_PAIRS_WG = 1024;      // gate/up pairs per workgroup
constexpr int D1_NB0 = 4;                  // first pass over h: 16-byte pieces per thread
constexpr int D1_MAX_LISTS = D1_NW;        // routing: experts E <= 64 * D1_MAX_LISTS

struct D1Plan {
    int G;              // workgroups
    int P;              // gate/up pairs of the layer
    int rw;             // output rows per workgroup
    uint64_t magic_rw;  // d / rw == (d * magic_rw) >> 32 for the small d used here
    int lpr_d;          // lanes per row of the down projection (down_lanes_per_row)
};

// First pair of workgroup w (even, so the two elements of an h word never
// belong to different workgroups)
__host__ __device__ inline int d1_pair_lo(int P, int G, int w) { return 2 * (int)(((int64_t)(P / 2) * w) / G); }

constexpr int D1_MAX_GROUPS = 33;           // k <= 32 routed + shared
constexpr int D1_H_LDS_WORDS = 16384;       // all of h as bf16 hi/lo words (64 KiB)
constexpr int D1_MAX_RW = 64;

struct D1Shared {
    int sel[D1_MAX_GROUPS];         // expert of group g (-1: shared)
    float wsel[D1_MAX_GROUPS];      // its gate weight (1 for the shared expert)
    u32 tag;
    u32 stale[3][2];                // per fetch round (mod 3): groups with a stale word
    __attribute__((aligned(16))) uint64_t lkey[D1_MAX_LISTS][64];   // routing: every expert's key, per wave
    __attribute__((aligned(16))) uint64_t cand[D1_MAX_LISTS * 32];  // routing: each wave's top-k keys
    uint64_t ranked[32];                // routing: the top-k keys in rank order
    float y[D1_MAX_GROUPS * D1_MAX_RW];   // down results: [group][local row]
};

// Region of the workspace for this kernel: h as [group][Imax] 64-bit words,
// word i = (call tag << 32) | fp32 bits of h_i.
__host__ __device__ inline size_t d1_h_offset(int H, int I, int Ish) {
    const size_t Imax = (size_t)(I > Ish ? I : Ish);
    return WS_HEADER + (size_t)DEC_MAX_PAIRS * Imax * 4 + (size_t)DEC_MAX_PAIRS * H * 4;
}

// Number of the N keys at p (LDS, 16-byte aligned) larger than key: all N/2
// 16-byte reads issued before any compare (every lane reads the same address).
template <int N>
__device__ inline int d1_count_greater(const uint64_t *p, uint64_t key) {
    const uint4 *q = reinterpret_cast<const uint4 *>(p);
    uint4 v[N / 2];
#pragma unroll
    for (int i = 0; i < N / 2; ++i) v[i] = q[i];
    int c = 0;
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
        const uint64_t a = ((uint64_t)v[i].y << 32) | v[i].x, b = ((uint64_t)v[i].w << 32) | v[i].z;
        c += (a > key) + (b > key);
    }
    return c;
}

// Number of the n (even) keys at p (LDS, 16-byte aligned) larger than key.
__device__ inline int d1_count_greater_list(const uint64_t *p, int n, uint64_t key) {
    const uint4 *q = reinterpret_cast<const uint4 *>(p);
    int c = 0;
#pragma unroll 8
    for (int i = 0; i < n / 2; ++i) {
        const uint4 v = q[i];
        const uint64_t a = ((uint64_t)v.y << 32) | v.x, b = ((uint64_t)v.w << 32) | v.z;
        c += (a > key) + (b > key);
    }
    return c;
}

// LDS layout of h: the 8 16-byte pieces of unit u are stored rotated by
// (u >> 1) & 7, so the 16 lanes of a row reading units u .. u+15 at the same
// piece hit 16 different bank groups.
__device__ inline int d1_piece_swz(int u) { return (u >> 1) & 7; }

template <int FMT, int DEC, int QG, int QD, int MG, int MD>
__global__ __launch_bounds__(D1_THREADS) void decode1_kernel(DecodeArgs a, D1Plan plan) {
    constexpr int PAIR = (DEC == DEC_LUT) ? (Fmt<FMT>::SIX ? LUT_E2M3_PAIR : LUT_E2M1_PAIR) : 1;
    __shared__ u32 s_pair[PAIR];
    __shared__ float s_scale[LUT_SCALE];
    __shared__ D1Shared S;
    extern __shared__ __attribute__((aligned(16))) u32 s_h[];   // NG * Imax words
    const Luts Lt{s_pair, s_scale};
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const LayerArgs &ly = a.L;
    const int H = ly.H, I = ly.I, k = ly.k, Ish = ly.Ish, E = ly.E;
    const int NG = k + (Ish > 0 ? 1 : 0);
    const int Imax = I > Ish ? I : Ish;
    u32 *hdr = reinterpret_cast<u32 *>(a.ws);
    uint64_t *hq = reinterpret_cast<uint64_t *>(a.ws + d1_h_offset(H, I, Ish));
    const int64_t crbH = Fmt<FMT>::code_row_bytes(H), srbH = Fmt<FMT>::scale_row_bytes(H);

    // call tag, activation units and the routing logits are all fetched at
    // once: wave w < NWL loads the logits of experts 64w .. 64w + 63
    const int NWL = (E + WAVE - 1) / WAVE;
    float lg1 = 0.f;
    if (wv < NWL) lg1 = a.logits[min(WAVE * wv + lane, E - 1)];
    if (tid == 64) S.tag = d1_ld_relaxed(&hdr[WS_EPOCH]) + 1u;
    if (tid >= 128 && tid < 134) (&S.stale[0][0])[tid - 128] = 0u;
    if (wv > 0) build_luts<FMT>(Lt, tid - 64, D1_THREADS - 64, DEC == DEC_LUT);
    const int UH = H / 32, LPRg = lanes_per_row(UH), RPWg = WAVE / LPRg;
    const int lrg = lane & (LPRg - 1), rsg = lane / LPRg;
    u32 xr[QG][1][16];
    {
        const uint16_t *xp[1] = {a.x};
        load_x_units<QG, 1>(xr, xp, UH, lrg, LPRg);
    }

    // ------------------------------------------------ route (every workgroup), by ranks
    // Every expert has a unique 64-bit key (larger key: larger logit, or the
    // same logit and a lower index), so its rank is the number of larger keys.
    // Level 1: wave w < NWL ranks its 64 experts among themselves (all compares
    // in parallel, no serial rounds) and lists those of rank < k.  Level 2: the
    // NWL * k listed keys are ranked among themselves; rank r < k is the
    // expert of rank r overall.
    const int KS = (k + 1) & ~1;   // list stride (even: 16-byte pair reads)
    if (wv < NWL) {
        const uint64_t key = expert_key(lg1, WAVE * wv + lane, WAVE * wv + lane < E);
        S.lkey[wv][lane] = key;
        __builtin_amdgcn_wave_barrier();   // the wave's own LDS writes precede its reads
        const int rank = d1_count_greater<WAVE>(S.lkey[wv], key);
        if (rank < k) S.cand[wv * KS + rank] = key;
        if (lane == 0 && KS > k) S.cand[wv * KS + k] = 0ull;   // padding: below every key
    }
    __syncthreads();
    {
        // candidate c's global rank: the sum over the lists of how many of
        // their keys are larger (exact for the top k: fewer than k keys of any
        // list are larger than such a candidate, so all of them are listed);
        // GS adjacent lanes take one candidate, one list each
        const int nc = NWL * KS;
        const int GS = NWL <= 1 ? 1 : NWL <= 2 ? 2 : NWL <= 4 ? 4 : NWL <= 8 ? 8 : 16;
        for (int t0 = 0; t0 < nc * GS; t0 += D1_THREADS) {
            const int t = t0 + tid, c = t / GS, wl = t - c * GS;
            uint64_t key = 0;
            int cnt = 0;
            if (c < nc) {
                key = S.cand[c];
                if (wl < NWL) cnt = d1_count_greater_list(S.cand + wl * KS, KS, key);
            }
            for (int off = GS >> 1; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
            if (c < nc && wl == 0 && (c % KS) < k && cnt < k) S.ranked[cnt] = key;
        }
    }
    __syncthreads();
    if (wv == 0) {
        int e;
        float wt;
        weights_from_ranked(lane < k ? S.ranked[lane] : 0ull, k, lane, e, wt);
        if (lane < k) {
            S.sel[lane] = e;
            S.wsel[lane] = wt;
            if (blockIdx.x == 0) {
                if (a.idx_out) a.idx_out[lane] = e;
                if (a.w_out) a.w_out[lane] = wt;
            }
        }
        if (lane == 0 && Ish > 0) {
            S.sel[k] = -1;
            S.wsel[k] = 1.0f;
        }
    }
    __syncthreads();

    // ------------------------------------------------ gate/up rows of this workgroup's pairs
    // slot s of a lane group holds pair j = (wave + 16 * (s / 2)) * RPWg + group,
    // its gate row in even slots and its up row in odd ones; pair pl + j belongs
    // to group min(p / I, k) (routed experts in rank order, then the shared one)
    const int w = blockIdx.x;
    const int pl = d1_pair_lo(plan.P, plan.G, w), n = d1_pair_lo(plan.P, plan.G, w + 1) - pl;
    static_assert(MG % 2 == 0, "gate and up slots come in pairs");
    Unit<FMT> gu_un[MG][QG];
#pragma unroll
    for (int s = 0; s < MG; ++s) {
        const int j = (wv + D1_NW * (s >> 1)) * RPWg + rsg;
        const int p = pl + (j < n ? j : 0);   // idle slots re-load pair 0
        const int g = min(p / I, k);
        const int i = p - g * I;
        const int e = S.sel[g];
        const int row = (s & 1) ? ((g < k) ? I : Ish) + i : i;
        // branch-free address selection (a branch here makes the compiler wait for loads in flight)
        const int64_t er = (int64_t)max(e, 0) * 2 * I + row;
        const uint8_t *c = (e >= 0 ? ly.w13c + er * crbH : ly.sh13c + (int64_t)row * crbH);
        const uint8_t *sc = (e >= 0 ? ly.w13s + er * srbH : ly.sh13s + (int64_t)row * srbH);
#pragma unroll
        for (int q = 0; q < QG; ++q) {
            const int u = lrg + LPRg * q;
            load_unit<FMT>(gu_un[s][q], c, sc, u < UH ? u : lrg);
        }
    }
    const int o0 = w * plan.rw;
    const int nr = max(0, min(H, o0 + plan.rw) - o0);

    // ---------------------------------------------- gate | up dots; each pair's h published at once
    const u32 tag = S.tag;
#pragma unroll
    for (int s2 = 0; s2 < MG / 2; ++s2) {
        float acc[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int s = 2 * s2 + h;
            acc[h] = 0.f;
#pragma unroll
            for (int q = 0; q < QG; ++q) {
                const int u = lrg + LPRg * q;
                if (u < UH) {
                    u32 wd[16];
                    decode_unit<FMT, DEC>(gu_un[s][q], Lt, wd);
                    float s0, s1;
                    unit_scales<FMT>(gu_un[s][q], Lt, s0, s1);
                    acc[h] = unit_dot<FMT>(wd, xr[q][0], s0, s1, acc[h]);
                }
            }
            acc[h] = group_sum_dpp(acc[h], LPRg);
        }
        const int j = (wv + D1_NW * s2) * RPWg + rsg;
        if (j < n && lrg == 0) {
            const float hv = silu_f32(acc[0]) * acc[1];
            const int p = pl + j, g = min(p / I, k), i = p - g * I;
            __hip_atomic_store(hq + (size_t)g * Imax + i, ((uint64_t)tag << 32) | __builtin_bit_cast(u32, hv),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    ring_barrier();   // this workgroup's h is published

    // ---------------------------------------------- first pass over all of h, then the down rows
    // Group g's words are Ig/2 16-byte pieces (two elements each), at piece
    // slots g*Imax/2 ...  The first pass
    // reads every slot once (D1_NB0 pieces per thread, ordinary loads: the
    // workgroups of an XCD share the lines through its L2); a piece whose two
    // tags are current goes to LDS, otherwise its group is read again.  The
    // down rows are issued after the first pass: h is on the critical path,
    // the down rows are not needed before it is complete.
    typedef __attribute__((ext_vector_type(4))) u32 v4u;
    const __amdgpu_buffer_rsrc_t hr = rsrc_of(hq, (uint64_t)NG * Imax * 8);
    const int slot_pc = Imax / 2;
    auto keep_piece = [&](int g, int pi, const v4u &pc, uint64_t &stale) {
        if (pc.y == tag && pc.w == tag) {
            // elements 2*pi, 2*pi + 1: their bf16 hi pair and lo pair words go to
            // unit u = pi / 16, pair pe = pi % 16 (hi in pieces 0..3, lo in 4..7, swizzled)
            // (components copied to scalars first: this compiler reads component 0
            // for a __builtin_bit_cast of a vector component)
            const u32 b0 = pc.x, b1 = pc.z;
            const float h0 = __builtin_bit_cast(float, b0), h1 = __builtin_bit_cast(float, b1);
            const u32 hi0 = f32_to_bf16_rne(h0), hi1 = f32_to_bf16_rne(h1);
            const u32 lo0 = f32_to_bf16_rne(h0 - __builtin_bit_cast(float, hi0 << 16));
            const u32 lo1 = f32_to_bf16_rne(h1 - __builtin_bit_cast(float, hi1 << 16));
            const int u = pi >> 4, pe = pi & 15, sw = d1_piece_swz(u);
            u32 *ub = s_h + g * Imax + 32 * u + (pe & 3);
            ub[4 * ((pe >> 2) ^ sw)] = hi0 | (hi1 << 16);
            ub[4 * ((4 + (pe >> 2)) ^ sw)] = lo0 | (lo1 << 16);
        } else {
            stale |= 1ull << g;
        }
    };
    v4u pc0[D1_NB0];
#pragma unroll
    for (int b = 0; b < D1_NB0; ++b) {
        const int q = tid + D1_THREADS * b, g = q / slot_pc, pi = q - g * slot_pc;
        const bool ok = g < NG && pi < ((g < k) ? I : Ish) / 2;
        pc0[b] = __builtin_amdgcn_raw_buffer_load_b128(hr, ok ? (int)(g * Imax * 8 + pi * 16) : 0, 0, 0);
    }

    const int LPRd = plan.lpr_d, RPWd = WAVE / LPRd;
    const int lrd = lane & (LPRd - 1), rsd = lane / LPRd;
    int dn_g[MD], dn_r[MD];
    Unit<FMT> dn_un[MD][QD];
#pragma unroll
    for (int s = 0; s < MD; ++s) {
        // down task d in [0, NG*nr): group d / rw, local row d % rw; idle
        // slots re-load task 0 (group 0, first row)
        const int d = (wv + D1_NW * s) * RPWd + rsd;
        const int g = (int)(((uint64_t)(u32)d * plan.magic_rw) >> 32);
        const int r = d - g * plan.rw;
        const bool ok = (nr > 0) && (g < NG) && (r < nr);
        dn_g[s] = ok ? g : -1;
        dn_r[s] = ok ? r : 0;
        const int e = S.sel[ok ? g : 0], o = min(o0 + dn_r[s], H - 1);
        const int Ig = (e >= 0) ? I : Ish;
        const int64_t crbI = Fmt<FMT>::code_row_bytes(Ig), srbI = Fmt<FMT>::scale_row_bytes(Ig);
        const int64_t eo = (int64_t)max(e, 0) * H + o;   // branch-free, as for the gate/up rows
        const uint8_t *c = (e >= 0) ? ly.w2c + eo * crbI : ly.sh2c + (int64_t)o * crbI;
        const uint8_t *sc = (e >= 0) ? ly.w2s + eo * srbI : ly.sh2s + (int64_t)o * srbI;
        const int Ug = Ig / 32;
#pragma unroll
        for (int q = 0; q < QD; ++q) {
            const int u = lrd + LPRd * q;
            load_unit<FMT>(dn_un[s][q], c, sc, u < Ug ? u : lrd);
        }
    }

    {
        uint64_t stale = 0;
#pragma unroll
        for (int b = 0; b < D1_NB0; ++b) {
            const int q = tid + D1_THREADS * b, g = q / slot_pc, pi = q - g * slot_pc;
            if (g < NG && pi < ((g < k) ? I : Ish) / 2) keep_piece(g, pi, pc0[b], stale);
        }
        stale = (uint64_t)wave_or_u32((u32)stale) | ((uint64_t)wave_or_u32((u32)(stale >> 32)) << 32);
        if (lane == 0 && stale != 0) {
            __hip_atomic_fetch_or(&S.stale[0][0], (u32)stale, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            __hip_atomic_fetch_or(&S.stale[0][1], (u32)(stale >> 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
    }
    ring_barrier();

    // ---------------------------------------------- further passes, device-coherent, over the stale groups
    // Pending groups are dealt to quarters of the workgroup in turn (256
    // threads each), a thread taking pieces t, t + 256, ... of its group.
    {
        uint64_t pending = (uint64_t)S.stale[0][0] | ((uint64_t)S.stale[0][1] << 32);
        if (a.spin_limit == 0u) {   // the test hook: the bounded wait expires at once
            if (tid == 0) d1_st_relaxed(&hdr[WS_ERR], 1u);
            pending = 0;
        }
        const int quarter = tid >> 8, qt = tid & 255;
        for (u32 round = 1; pending != 0; ++round) {
            if (round > a.spin_limit) {
                if (tid == 0) d1_st_relaxed(&hdr[WS_ERR], 1u);
                break;
            }
            if (tid == 0) { S.stale[(round + 1) % 3][0] = 0u; S.stale[(round + 1) % 3][1] = 0u; }
            __builtin_amdgcn_s_sleep(1);
            uint64_t stale = 0;
            int j = 0;
            for (uint64_t m = pending; m != 0; m &= m - 1, ++j) {
                if ((j & 3) != quarter) continue;
                const int g = __builtin_ctzll(m);
                const int npc = ((g < k) ? I : Ish) / 2;
                constexpr int NB = 2;
                for (int b0 = 0; b0 < npc; b0 += 256 * NB) {
                    v4u pc[NB];
#pragma unroll
                    for (int b = 0; b < NB; ++b) {
                        const int pi = b0 + 256 * b + qt;
                        pc[b] = __builtin_amdgcn_raw_buffer_load_b128(hr, (int)(g * Imax * 8 + (pi < npc ? pi : 0) * 16),
                                                                     0, 16);   // sc1
                    }
#pragma unroll
                    for (int b = 0; b < NB; ++b) {
                        const int pi = b0 + 256 * b + qt;
                        if (pi < npc) keep_piece(g, pi, pc[b], stale);
                    }
                }
            }
            stale = (uint64_t)wave_or_u32((u32)stale) | ((uint64_t)wave_or_u32((u32)(stale >> 32)) << 32);
            if (lane == 0 && stale != 0) {
                __hip_atomic_fetch_or(&S.stale[round % 3][0], (u32)stale, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                __hip_atomic_fetch_or(&S.stale[round % 3][1], (u32)(stale >> 32), __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_WORKGROUP);
            }
            ring_barrier();
            pending = (uint64_t)S.stale[round % 3][0] | ((uint64_t)S.stale[round % 3][1] << 32);
        }
    }

    // ---------------------------------------------- down dots
#pragma unroll
    for (int s = 0; s < MD; ++s) {
        float acc = 0.f;
        if (dn_g[s] >= 0) {
            const int g = dn_g[s];
            const int Ug = ((g < k) ? I : Ish) / 32;
#pragma unroll
            for (int q = 0; q < QD; ++q) {
                const int u = lrd + LPRd * q;
                if (u < Ug) {
                    const uint4 *hb = reinterpret_cast<const uint4 *>(s_h + g * Imax + 32 * u);
                    const int sw = d1_piece_swz(u);
                    u32 xh[16], xl[16];
#pragma unroll
                    for (int vv = 0; vv < 4; ++vv) {
                        const uint4 A = hb[vv ^ sw], B = hb[(4 + vv) ^ sw];
                        xh[4 * vv] = A.x; xh[4 * vv + 1] = A.y; xh[4 * vv + 2] = A.z; xh[4 * vv + 3] = A.w;
                        xl[4 * vv] = B.x; xl[4 * vv + 1] = B.y; xl[4 * vv + 2] = B.z; xl[4 * vv + 3] = B.w;
                    }
                    u32 wd[16];
                    decode_unit<FMT, DEC>(dn_un[s][q], Lt, wd);
                    float s0, s1;
                    unit_scales<FMT>(dn_un[s][q], Lt, s0, s1);
                    acc = unit_dot_split<FMT>(wd, xh, xl, s0, s1, acc);
                }
            }
        }
        acc = group_sum_dpp(acc, LPRd);
        if (dn_g[s] >= 0 && lrd == 0) S.y[dn_g[s] * D1_MAX_RW + dn_r[s]] = acc;
    }
    __syncthreads();
    for (int r = tid; r < nr; r += D1_THREADS) {
        float acc = 0.f;
#pragma unroll 8
        for (int g = 0; g < k; ++g) acc = __builtin_fmaf(S.wsel[g], S.y[g * D1_MAX_RW + r], acc);
        if (Ish > 0) acc += S.y[k * D1_MAX_RW + r];
        if (a.residual) acc += bf16_to_f32(a.residual[o0 + r]);
        if (a.out_f32) reinterpret_cast<float *>(a.out)[o0 + r] = acc;
        else reinterpret_cast<uint16_t *>(a.out)[o0 + r] = f32_to_bf16_rne(acc);
    }
    // every workgroup leaves its tag as the call counter (a max, so the counter
    // never moves back even after an expired wait)
    if (tid == 0) __hip_atomic_fetch_max(&hdr[WS_EPOCH], S.tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace moeq

namespace moeq {

// Workgroups of `kernel` that can be resident at once on the current device
// (cached per device and LDS size: no runtime query after the first call).
template <typename K>
static int d1_coresident(K kernel, size_t dyn_lds, int &cus) {
    cus = cached_cus();
    return cached_occupancy(reinterpret_cast<const void *>(kernel), D1_THREADS, dyn_lds) * cus;
}

// Try a launch with MG gate/up slots and MD down slots per wave; returns
// hipErrorNotSupported when the shape does not fit (the caller falls back).
template <int FMT, int DEC, int QG, int QD, int MG, int MD>
static hipError_t decode1_try(const DecodeArgs &a, hipStream_t s) {
    auto kern = decode1_kernel<FMT, DEC, QG, QD, MG, MD>;
    const LayerArgs &L = a.L;
    const int NG = L.k + (L.Ish > 0 ? 1 : 0);
    const int Imax = L.I > L.Ish ? L.I : L.Ish;
    const size_t dyn = (size_t)NG * Imax * 4;
    int cus = 0;
    const int cap = d1_coresident(kern, dyn, cus);
    const int RPWg = WAVE / lanes_per_row(L.H / 32);
    const int RPWd = WAVE / down_lanes_per_row(L.I, L.Ish);
    const int P = L.k * L.I + L.Ish;
    // one workgroup on 7/8 of the CUs (all must be resident: they wait on each
    // other), fewer for a small layer (at least 16 pairs each).  On the wide
    // layer (5,632 pairs, 256 CUs) 216-224 workgroups took 16.64 us against
    // 16.98 with all 256 and 17.86 with 192: fewer workgroups to wait for in
    // the h exchange, against more rows each.
    int G = cus - cus / 8;
    if (G > P / 16) G = P / 16;
    if (G > cap) G = cap;
    if (G < 1) return hipErrorNotSupported;
    int nmax = 0;   // the largest pair range
    for (int w = 0; w < G; ++w) nmax = std::max(nmax, d1_pair_lo(P, G, w + 1) - d1_pair_lo(P, G, w));
    if (nmax > D1_MAX_PAIRS_WG || nmax > D1_NW * (MG / 2) * RPWg) return hipErrorNotSupported;
    const int rw = (L.H + G - 1) / G;
    if (rw > D1_MAX_RW || NG * rw > D1_NW * MD * RPWd) return hipErrorNotSupported;
    // m = floor(2^32 / rw) + 1 = 2^32 / rw + f with 0 < f <= 1, so d * m / 2^32 =
    // d / rw + d * f / 2^32 and the floor is exact while d * f / 2^32 < 1 / rw,
    // i.e. for every d < 2^32 / rw: here d < 16 * 64 * MD (wave, lane group,
    // slot) and rw <= 64, far below that
    static_assert((uint64_t)D1_NW * 64 * MD * D1_MAX_RW < (1ull << 32), "magic division range");
    D1Plan plan{G, P, rw, (1ull << 32) / (uint64_t)rw + 1u, down_lanes_per_row(L.I, L.Ish)};
    hipLaunchKernelGGL(kern, dim3(G), dim3(D1_THREADS), dyn, s, a, plan);
    return hipGetLastError();
}

template <int FMT, int DEC, int QG, int QD>
static hipError_t decode1_q(const DecodeArgs &a, hipStream_t s) {
    hipError_t e = decode1_try<FMT, DEC, QG, QD, 2, 1>(a, s);
    if (e != hipErrorNotSupported) return e;
    e = decode1_try<FMT, DEC, QG, QD, 4, 2>(a, s);
    if (e != hipErrorNotSupported) return e;
    return decode1_try<FMT, DEC, QG, QD, 8, 4>(a, s);
}

template <int FMT, int DEC>
hipError_t decode1_fd(const DecodeArgs &a, hipStream_t s) {
    const LayerArgs &L = a.L;
    if (a.T != 1 || a.mode != MODE_ROUTE) return hipErrorNotSupported;
    const int NG = L.k + (L.Ish > 0 ? 1 : 0);
    const int Imax = L.I > L.Ish ? L.I : L.Ish;
    if (NG > D1_MAX_GROUPS || NG * Imax > D1_H_LDS_WORDS || NG * Imax / 2 > D1_NB0 * D1_THREADS ||
        L.E > WAVE * D1_MAX_LISTS)
        return hipErrorNotSupported;
    const int UH = L.H / 32, LPRg = lanes_per_row(UH), QG = (UH + LPRg - 1) / LPRg;
    const int LPRd = down_lanes_per_row(L.I, L.Ish), QD = (Imax / 32 + LPRd - 1) / LPRd;
    if (QG == 1 && QD == 1) return decode1_q<FMT, DEC, 1, 1>(a, s);
    if (QG == 1 && QD == 2) return decode1_q<FMT, DEC, 1, 2>(a, s);
    if (QG == 2 && QD == 1) return decode1_q<FMT, DEC, 2, 1>(a, s);
    if (QG == 2 && QD == 2) return decode1_q<FMT, DEC, 2, 2>(a, s);
    return hipErrorNotSupported;
}

}  // namespace moeq
