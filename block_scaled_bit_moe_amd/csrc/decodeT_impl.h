// decodeT_impl.h -- the MoE layer for 2..16 tokens in one launch (the decode
// step of nextsycl README, "What it does": gate | up and down expert kernels,
// several rows decoded together with each row exactly as its own pass; Strata
// docs/INTEL.md, "The engine itself on Intel": router_top10, shared_expert).
//
// One workgroup of 16 waves per CU (all resident), every one running the same
// four phases on static shares of the work, with no work items:
//   A. route every token (wave t routes token t) and build the expert groups
//      in LDS (ascending expert id, tokens ascending inside an expert, the
//      shared expert last with every token);
//   B. gate | up: the groups' row pairs (group-major) are split into G shares
//      of equal cost (a row pair of a group with m tokens costs its weight
//      bytes plus m dot products); a workgroup walks its share one group at a
//      time, with the group's tokens (up to DT_XT per batch) in LDS, deals the
//      row pairs to its waves from an LDS counter, streams each gate row and
//      its up row through one lane group, and publishes h of every (token,
//      row) as a 64-bit word (call tag << 32 | fp32 bits);
//   C. down: the groups' output rows are split the same way; per group, the
//      workgroup reads that group's h for a token batch (tagged words, read
//      again until every tag is current) into LDS as bf16 hi/lo pairs, streams
//      its down rows and publishes the partial outputs as tagged words;
//   D. combine: workgroup w owns output rows [w*RW, (w+1)*RW) of every token
//      and sums the partials of the token's experts in rank order (plus the
//      shared expert) once all their tags are current, then rounds once.
// Every row is computed with the same lane mapping, unit order and reduction
// as in the single-token kernel, so a token's result does not depend on the
// other tokens of the call or on which kernel ran it.  The tag is the
// workspace's call counter + 1, read on entry and raised on exit; a workgroup
// that started after another had already finished would carry a newer tag,
// and every wait on or of it would expire and be reported (no stale word is
// ever taken as current).
#pragma once

#include "decode1_impl.h"

namespace moeq {

constexpr int DT_NW = 16;
constexpr int DT_THREADS = 64 * DT_NW;
constexpr int DT_XT = 8;                          // most tokens of a batch (x or h in LDS)
constexpr size_t DT_LDS = 112 * 1024;            // dynamic LDS: one batch's x (gate/up) or h (down)
constexpr int DT_MAX_GROUPS = DEC_MAX_T * 32 + 1;
constexpr int DT_HPT = 8;                         // h pieces per thread per read pass (phase C)

// Rows per lane group and item (gate/up: row pairs), so that every lane has
// several unit loads in flight per item.
__host__ __device__ constexpr int dt_rows_gu(int QG) { return QG >= 2 ? 1 : 2; }
__host__ __device__ constexpr int dt_rows_dn(int QD) { return QD >= 2 ? 1 : 2; }

// Relative cost of one row (gate/up: one row pair) of a group with m tokens:
// streaming its weights plus m dot products.  The static split of each phase
// gives every workgroup an equal share of this cost rather than of the rows,
// so that workgroups holding experts with several tokens get fewer rows.  The
// constants are the ratios measured on a 6144-wide layer with 2048-wide
// experts (six-bit codes carry 6.25 instead of 4.5 bits per weight).
template <int FMT> __host__ __device__ constexpr int dt_cost_gu(int m) { return (Fmt<FMT>::SIX ? 8 : 6) + 2 * m; }
template <int FMT> __host__ __device__ constexpr int dt_cost_dn(int m) { return (Fmt<FMT>::SIX ? 4 : 3) + 2 * m; }

// The first group g with cum[g + 1] > c (cum ascending, cum[0] = 0, c < cum[n]).
__device__ inline int dt_first_group(const int *cum, int n, int c) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (cum[mid + 1] > c) hi = mid;
        else lo = mid + 1;
    }
    return lo;
}
// Rows r of a group whose cost position cum + r * cost falls below c: the
// ranges [row_at(c0), row_at(c1)) of consecutive shares partition the rows.
__device__ inline int dt_row_at(int c, int cost) { return c <= 0 ? 0 : (c + cost - 1) / cost; }

struct DTPlan {
    int G;       // workgroups
    int rw;      // output rows per workgroup (phase D)
    int xt_gu;   // tokens per batch in phase B
    int xt_dn;   // tokens per batch in phase C
};

struct DTShared {
    int idx[DEC_MAX_T * 32];
    float w[DEC_MAX_T * 32];
    u32 tmask[1024];                      // tokens of each expert (bit t)
    short e2g[1024];
    short g_expert[DT_MAX_GROUPS];        // -1: the shared expert
    short g_start[DT_MAX_GROUPS];         // first pair position
    unsigned char g_count[DT_MAX_GROUPS];
    unsigned char p_tok[DEC_MAX_PAIRS];   // token of each pair position
    short pos_of[DEC_MAX_T][33];          // pair position of (token, rank); rank k: the shared expert
    int scan[2 * DT_NW];
    int n_groups;
    u32 tag;
    int next[2];                          // work counters of even / odd batches
    int cum_gu[DT_MAX_GROUPS + 1];        // cost of the groups before g (gate/up, down)
    int cum_dn[DT_MAX_GROUPS + 1];
};

// Workspace regions of this kernel (after those of the other decode kernels):
// h as [pair][Imax] and partial outputs as [pair][H], tagged 64-bit words.
__host__ __device__ inline size_t dt_h_offset(int H, int I, int Ish) {
    const size_t Imax = (size_t)(I > Ish ? I : Ish);
    return d1_h_offset(H, I, Ish) + (size_t)33 * Imax * 8;
}
__host__ __device__ inline size_t dt_y_offset(int H, int I, int Ish) {
    const size_t Imax = (size_t)(I > Ish ? I : Ish);
    return dt_h_offset(H, I, Ish) + (size_t)DEC_MAX_PAIRS * Imax * 8;
}

// A tagged word (tag << 32 | fp32 bits) at byte offset voff + soff, written
// with one 64-bit store through to the device coherence point (sc1), as the
// single-token kernel's h words are.  The uniform part of the offset goes in
// the instruction's scalar offset.
__device__ inline void dt_store_tagged(__amdgpu_buffer_rsrc_t r, u32 voff, u32 soff, u32 tag, float v) {
    typedef __attribute__((ext_vector_type(2))) u32 v2u;
    v2u d;
    d.x = __builtin_bit_cast(u32, v);
    d.y = tag;
    __builtin_amdgcn_raw_buffer_store_b64(d, r, (int)voff, (int)soff, 16);
}

// exclusive scan of two counters over the 1024 threads
__device__ inline void dt_exscan2(int a, int b, int &ea, int &eb, int &ta, int &tb, int *tmp) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int ia = a, ib = b;
    for (int m = 1; m < 64; m <<= 1) {
        const int oa = __shfl_up(ia, m, WAVE), ob = __shfl_up(ib, m, WAVE);
        if (lane >= m) { ia += oa; ib += ob; }
    }
    if (lane == 63) { tmp[wv] = ia; tmp[DT_NW + wv] = ib; }
    __syncthreads();
    int pa = 0, pb = 0;
    ta = 0;
    tb = 0;
    for (int v = 0; v < DT_NW; ++v) {
        if (v < wv) { pa += tmp[v]; pb += tmp[DT_NW + v]; }
        ta += tmp[v];
        tb += tmp[DT_NW + v];
    }
    ea = pa + ia - a;
    eb = pb + ib - b;
    __syncthreads();
}

// Activations in LDS, unit-major: unit u of token slot t at word u * US + t * W
// (W = 16 words of bf16 x, or 32 words of h as 16 hi + 16 lo), where the unit
// stride US = W * slots + 4 words.  The 4-word pad puts 16 consecutive units
// on 16 different groups of 4 banks, and a lane's reads of every token and
// piece of its unit are one base address plus immediate offsets.
__host__ __device__ inline int dt_unit_stride(int W, int slots) { return W * slots + 4; }
__host__ __device__ inline size_t dt_lds_bytes(int units, int W, int slots) {
    return (size_t)units * dt_unit_stride(W, slots) * 4;
}

// XT: tokens per batch (4 or 8).  Four keep the per-row accumulators small
// (measured on the batched layer: 467 against 481 us); eight halve the
// number of passes over a group's rows when it has more than four tokens,
// which a shared expert always has at T > 4.
template <int FMT, int DEC, int QG, int QD, int XT>
__global__ __launch_bounds__(DT_THREADS) void decodeT_kernel(DecodeArgs a, DTPlan plan) {
    constexpr int PAIR = (DEC == DEC_LUT) ? (Fmt<FMT>::SIX ? LUT_E2M3_PAIR : LUT_E2M1_PAIR) : 1;
    __shared__ u32 s_pair[PAIR];
    __shared__ float s_scale[LUT_SCALE];
    __shared__ DTShared S;
    extern __shared__ __attribute__((aligned(16))) u32 s_buf[];
    const Luts Lt{s_pair, s_scale};
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const LayerArgs &ly = a.L;
    const int H = ly.H, I = ly.I, k = ly.k, Ish = ly.Ish, E = ly.E, T = a.T;
    const int Imax = I > Ish ? I : Ish;
    const int w = blockIdx.x, G = plan.G;
    u32 *hdr = reinterpret_cast<u32 *>(a.ws);
    uint64_t *hq = reinterpret_cast<uint64_t *>(a.ws + dt_h_offset(H, I, Ish));
    uint64_t *yq = reinterpret_cast<uint64_t *>(a.ws + dt_y_offset(H, I, Ish));
    const int64_t crbH = Fmt<FMT>::code_row_bytes(H), srbH = Fmt<FMT>::scale_row_bytes(H);
    typedef __attribute__((ext_vector_type(4))) u32 v4u;

    // ------------------------------------------------ A. route, expert groups
    if (tid == 0) {
        S.tag = d1_ld_relaxed(&hdr[WS_EPOCH]) + 1u;
        S.next[0] = 0;
        S.next[1] = 0;
    }
    build_luts<FMT>(Lt, tid, DT_THREADS, DEC == DEC_LUT);
    for (int e = tid; e < 1024; e += DT_THREADS) S.tmask[e] = 0u;
    if (wv < T) {
        const int t = wv;
        int e;
        float wt;
        const float *lg = a.logits + (int64_t)t * E;
        if (E <= 64) route_one_token_wave<1>(lg, E, k, lane, e, wt);
        else if (E <= 128) route_one_token_wave<2>(lg, E, k, lane, e, wt);
        else if (E <= 256) route_one_token_wave<4>(lg, E, k, lane, e, wt);
        else if (E <= 512) route_one_token_wave<8>(lg, E, k, lane, e, wt);
        else route_one_token_wave<16>(lg, E, k, lane, e, wt);
        if (lane < k) {
            S.idx[t * k + lane] = e;
            S.w[t * k + lane] = wt;
            if (blockIdx.x == 0) {
                if (a.idx_out) a.idx_out[(int64_t)t * k + lane] = e;
                if (a.w_out) a.w_out[(int64_t)t * k + lane] = wt;
            }
        }
    }
    __syncthreads();
    for (int p = tid; p < T * k; p += DT_THREADS) atomicOr(&S.tmask[S.idx[p]], 1u << (p / k));
    __syncthreads();
    {
        const int e = tid;
        const u32 m = (e < E) ? S.tmask[e] : 0u;
        int ef, ec, nf, nc;
        dt_exscan2(m != 0u, __builtin_popcount(m), ef, ec, nf, nc, S.scan);
        // the costs are affine in m, so their prefix over the routed groups follows from the same scan
        constexpr int gu0 = dt_cost_gu<FMT>(0), gu1 = dt_cost_gu<FMT>(1) - gu0;
        constexpr int dn0 = dt_cost_dn<FMT>(0), dn1 = dt_cost_dn<FMT>(1) - dn0;
        if (m != 0u) {
            S.e2g[e] = (short)ef;
            S.g_expert[ef] = (short)e;
            S.g_start[ef] = (short)ec;
            S.g_count[ef] = (unsigned char)__builtin_popcount(m);
            S.cum_gu[ef] = I * (gu0 * ef + gu1 * ec);
            S.cum_dn[ef] = H * (dn0 * ef + dn1 * ec);
            u32 mm = m;
            for (int n = 0; mm; ++n) {
                S.p_tok[ec + n] = (unsigned char)__builtin_ctz(mm);
                mm &= mm - 1u;
            }
        }
        if (tid == 0) {
            S.n_groups = nf + (Ish > 0 ? 1 : 0);
            int cg = I * (gu0 * nf + gu1 * nc), cd = H * (dn0 * nf + dn1 * nc);
            if (Ish > 0) {
                S.g_expert[nf] = -1;
                S.g_start[nf] = (short)nc;
                S.g_count[nf] = (unsigned char)T;
                S.cum_gu[nf] = cg;
                S.cum_dn[nf] = cd;
                cg += Ish * dt_cost_gu<FMT>(T);
                cd += H * dt_cost_dn<FMT>(T);
            }
            S.cum_gu[S.n_groups] = cg;
            S.cum_dn[S.n_groups] = cd;
        }
        if (Ish > 0 && tid < T) S.p_tok[nc + tid] = (unsigned char)tid;
        if (Ish > 0 && tid < T) S.pos_of[tid][k] = (short)(nc + tid);
    }
    __syncthreads();
    // pair position of every (token, rank); read only by the combine, after a later barrier
    for (int p = tid; p < T * k; p += DT_THREADS) {
        const int t = p / k, r = p - t * k, e = S.idx[p];
        S.pos_of[t][r] = (short)(S.g_start[S.e2g[e]] + __builtin_popcount(S.tmask[e] & ((1u << t) - 1u)));
    }
    const int NG = S.n_groups;
    const u32 tag = S.tag;
    // Work inside a batch (one group's row range and up to XT of its tokens)
    // is dealt to the waves one item at a time from an LDS counter, so that a
    // wave that gets its loads served sooner takes more items and all waves
    // finish together.  Batches alternate between two counters: batch n+1's is
    // cleared after the barrier that opens batch n, when no wave can still
    // take from it (its last use was batch n-1).
    int nbatch = 0;
    auto open_batch = [&]() {
        if (tid == 0) S.next[(nbatch + 1) & 1] = 0;
    };
    auto grab = [&]() -> int {
        int v = 0;
        if (lane == 0) v = atomicAdd(&S.next[nbatch & 1], 1);
        return __builtin_amdgcn_readfirstlane(v);
    };

    // ------------------------------------------------ B. gate | up, h published
    {
        const int UH = H / 32, LPRg = lanes_per_row(UH), RPWg = WAVE / LPRg;
        const int lrg = lane & (LPRg - 1), rsg = lane / LPRg;
        const int USx = dt_unit_stride(16, plan.xt_gu);
        const __amdgpu_buffer_rsrc_t hw = rsrc_of(hq, (uint64_t)DEC_MAX_PAIRS * Imax * 8);
        const int c0 = (int)((int64_t)S.cum_gu[NG] * w / G), c1 = (int)((int64_t)S.cum_gu[NG] * (w + 1) / G);
        for (int g = dt_first_group(S.cum_gu, NG, c0); g < NG && S.cum_gu[g] < c1; ++g) {
            const int e = S.g_expert[g], m = S.g_count[g], pos0 = S.g_start[g], Ig = (e >= 0) ? I : Ish;
            const int cost = dt_cost_gu<FMT>(m);
            const int i0 = dt_row_at(c0 - S.cum_gu[g], cost), i1 = min(Ig, dt_row_at(c1 - S.cum_gu[g], cost));
            if (i0 >= i1) continue;
            const int nsub = i1 - i0;
            const uint8_t *c13 = (e >= 0) ? ly.w13c + (int64_t)max(e, 0) * 2 * I * crbH : ly.sh13c;
            const uint8_t *s13 = (e >= 0) ? ly.w13s + (int64_t)max(e, 0) * 2 * I * srbH : ly.sh13s;
            constexpr int RG = dt_rows_gu(QG);
            const int nitem = (nsub + RG * RPWg - 1) / (RG * RPWg);
            // row pair b of item it for this lane group
            auto jrow = [&](int it, int b) { return (it * RG + b) * RPWg + rsg; };
            for (int tb = 0; tb < m; tb += plan.xt_gu) {
                const int mb = min(plan.xt_gu, m - tb);
                __syncthreads();   // the previous batch is done with s_buf and its counter
                open_batch();
                for (int q = tid; q < mb * UH * 4; q += DT_THREADS) {
                    const int t = q / (UH * 4), rem = q - t * (UH * 4), u = rem >> 2, v = rem & 3;
                    const uint4 val = *reinterpret_cast<const uint4 *>(a.x + (int64_t)S.p_tok[pos0 + tb + t] * H + 32 * u + 8 * v);
                    *reinterpret_cast<uint4 *>(s_buf + u * USx + 16 * t + 4 * v) = val;
                }
                __syncthreads();
                Unit<FMT> un[1][RG][2][QG];
                auto issue = [&](int st, int p) {
#pragma unroll
                    for (int b = 0; b < RG; ++b) {
                        const int j = jrow(p, b);
                        const int r = i0 + (j < nsub ? j : 0);   // past the end: re-load the first row
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const int row = h ? Ig + r : r;
                            const uint8_t *c = c13 + (int64_t)row * crbH, *sc = s13 + (int64_t)row * srbH;
#pragma unroll
                            for (int q = 0; q < QG; ++q) {
                                const int u = lrg + LPRg * q;
                                load_unit<FMT>(un[st][b][h][q], c, sc, u < UH ? u : lrg);
                            }
                        }
                    }
                };
                auto compute = [&](int st, int p) {
#pragma unroll
                    for (int b = 0; b < RG; ++b) {
                        float acc[2][XT];
#pragma unroll
                        for (int h = 0; h < 2; ++h)
#pragma unroll
                            for (int t = 0; t < XT; ++t) acc[h][t] = 0.f;
#pragma unroll
                        for (int h = 0; h < 2; ++h)
#pragma unroll
                            for (int q = 0; q < QG; ++q) {
                                const int u = lrg + LPRg * q;
                                u32 wd[16];
                                decode_unit<FMT, DEC>(un[st][b][h][q], Lt, wd);
                                float s0, s1;
                                unit_scales<FMT>(un[st][b][h][q], Lt, s0, s1);
                                const int uu = u < UH ? u : 0;
                                const uint4 *xb = reinterpret_cast<const uint4 *>(s_buf + uu * USx);
#pragma unroll
                                for (int t = 0; t < XT; ++t) {
                                    if (t < mb) {
                                        const uint4 *xt = xb + 4 * t;
                                        u32 xv[16];
#pragma unroll
                                        for (int v = 0; v < 4; ++v) {
                                            const uint4 A = xt[v];
                                            xv[4 * v] = A.x; xv[4 * v + 1] = A.y; xv[4 * v + 2] = A.z; xv[4 * v + 3] = A.w;
                                        }
                                        const float d = unit_dot<FMT>(wd, xv, s0, s1, acc[h][t]);
                                        acc[h][t] = u < UH ? d : acc[h][t];
                                    }
                                }
                            }
                        const int j = jrow(p, b);
#pragma unroll
                        for (int t = 0; t < XT; ++t) {
                            if (t < mb) {
                                const float gsum = group_sum_dpp(acc[0][t], LPRg), usum = group_sum_dpp(acc[1][t], LPRg);
                                if (j < nsub && lrg == 0) {
                                    const float hv = silu_f32(gsum) * usum;
                                    dt_store_tagged(hw, (u32)(i0 + j) * 8u, (u32)((pos0 + tb + t) * Imax) * 8u, tag, hv);
                                }
                            }
                        }
                    }
                };
                // one item per wave at a time (the other waves' loads cover the
                // wait): on the batched layer 0.455 ms against 0.461 with the next
                // item's loads in flight during the dots (fewer rows open per CU
                // stream faster; the down phase below keeps two in flight, which
                // measured faster there).  An item past the end loads the first
                // rows again.
                int ia = grab();
                issue(0, ia);
                for (;;) {
                    if (ia >= nitem) break;
                    compute(0, ia);
                    ia = grab();
                    issue(0, ia);
                }
                ++nbatch;
            }
        }
    }

    // ------------------------------------------------ C. down, partial outputs published
    // Bounded waits (a thread's waits share one budget of spin_limit polls);
    // spin_limit 0 is the test hook: the wait expires at once, reported.
    u32 spins = 0;
    if (a.spin_limit == 0u && tid == 0) d1_st_relaxed(&hdr[WS_ERR], 1u);
    {
        const int LPRd = down_lanes_per_row(I, Ish), RPWd = WAVE / LPRd;
        const int lrd = lane & (LPRd - 1), rsd = lane / LPRd;
        const int USh = dt_unit_stride(32, plan.xt_dn);
        const __amdgpu_buffer_rsrc_t yw = rsrc_of(yq, (uint64_t)DEC_MAX_PAIRS * H * 8);
        const __amdgpu_buffer_rsrc_t hr = rsrc_of(hq, (uint64_t)DEC_MAX_PAIRS * Imax * 8);
        const int c0 = (int)((int64_t)S.cum_dn[NG] * w / G), c1 = (int)((int64_t)S.cum_dn[NG] * (w + 1) / G);
        for (int g = dt_first_group(S.cum_dn, NG, c0); g < NG && S.cum_dn[g] < c1; ++g) {
            const int e = S.g_expert[g], m = S.g_count[g], pos0 = S.g_start[g];
            const int cost = dt_cost_dn<FMT>(m);
            const int o0 = dt_row_at(c0 - S.cum_dn[g], cost), o1 = min(H, dt_row_at(c1 - S.cum_dn[g], cost));
            if (o0 >= o1) continue;
            const int nsub = o1 - o0;
            const int Ig = (e >= 0) ? I : Ish, UI = Ig / 32;
            const int64_t crbI = Fmt<FMT>::code_row_bytes(Ig), srbI = Fmt<FMT>::scale_row_bytes(Ig);
            const uint8_t *c2 = (e >= 0) ? ly.w2c + (int64_t)max(e, 0) * H * crbI : ly.sh2c;
            const uint8_t *s2 = (e >= 0) ? ly.w2s + (int64_t)max(e, 0) * H * srbI : ly.sh2s;
            constexpr int RD = dt_rows_dn(QD);
            const int nitem = (nsub + RD * RPWd - 1) / (RD * RPWd);
            // row b of item it for this lane group
            auto jrow = [&](int it, int b) { return (it * RD + b) * RPWd + rsd; };
            for (int tb = 0; tb < m; tb += plan.xt_dn) {
                const int mb = min(plan.xt_dn, m - tb);
                Unit<FMT> un[2][RD][QD];
                auto issue = [&](int st, int p) {
#pragma unroll
                    for (int b = 0; b < RD; ++b) {
                        const int j = jrow(p, b);
                        const int o = o0 + (j < nsub ? j : 0);
                        const uint8_t *c = c2 + (int64_t)o * crbI, *sc = s2 + (int64_t)o * srbI;
#pragma unroll
                        for (int q = 0; q < QD; ++q) {
                            const int u = lrd + LPRd * q;
                            load_unit<FMT>(un[st][b][q], c, sc, u < UI ? u : lrd);
                        }
                    }
                };
                __syncthreads();   // the previous batch is done with s_buf and its counter
                open_batch();
                int ia = grab();
                issue(0, ia);      // the weights do not depend on h: in flight during its wait
                // h of this batch: token t's Ig/2 pieces of two tagged words, into LDS as hi/lo pairs
                {
                    const int npc = mb * (Ig / 2);
                    u32 stale = 0;
                    auto put = [&](int q, const v4u &pc) {
                        const u32 b0 = pc.x, b1 = pc.z;   // (scalars first: see the single-token kernel)
                        if (pc.y != tag || pc.w != tag) return false;
                        const int t = q / (Ig / 2), pi = q - t * (Ig / 2);
                        const float h0 = __builtin_bit_cast(float, b0), h1 = __builtin_bit_cast(float, b1);
                        const u32 hi0 = f32_to_bf16_rne(h0), hi1 = f32_to_bf16_rne(h1);
                        const u32 lo0 = f32_to_bf16_rne(h0 - __builtin_bit_cast(float, hi0 << 16));
                        const u32 lo1 = f32_to_bf16_rne(h1 - __builtin_bit_cast(float, hi1 << 16));
                        const int u = pi >> 4, pe = pi & 15;
                        u32 *ub = s_buf + u * USh + 32 * t + pe;
                        ub[0] = hi0 | (hi1 << 16);
                        ub[16] = lo0 | (lo1 << 16);
                        return true;
                    };
                    auto src = [&](int q) {
                        const int t = q / (Ig / 2), pi = q - t * (Ig / 2);
                        return (u32)(((size_t)(pos0 + tb + t) * Imax) * 8 + pi * 16);
                    };
                    v4u pc[DT_HPT];
#pragma unroll
                    for (int b = 0; b < DT_HPT; ++b) {
                        const int q = tid + DT_THREADS * b;
                        pc[b] = __builtin_amdgcn_raw_buffer_load_b128(hr, (int)(q < npc ? src(q) : 0u), 0, 0);
                    }
#pragma unroll
                    for (int b = 0; b < DT_HPT; ++b) {
                        const int q = tid + DT_THREADS * b;
                        if (q < npc && !put(q, pc[b])) stale |= 1u << b;
                    }
                    while (stale != 0u) {
                        if (spins >= a.spin_limit) {
                            d1_st_relaxed(&hdr[WS_ERR], 1u);
                            break;
                        }
                        ++spins;
                        __builtin_amdgcn_s_sleep(1);
                        for (u32 m2 = stale; m2 != 0u; m2 &= m2 - 1u) {
                            const int b = __builtin_ctz(m2), q = tid + DT_THREADS * b;
                            const v4u p1 = __builtin_amdgcn_raw_buffer_load_b128(hr, (int)src(q), 0, 16);   // sc1
                            if (put(q, p1)) stale &= ~(1u << b);
                        }
                    }
                }
                __syncthreads();
                auto compute = [&](int st, int it) {
                    float acc[RD][XT];
#pragma unroll
                    for (int b = 0; b < RD; ++b)
#pragma unroll
                        for (int t = 0; t < XT; ++t) acc[b][t] = 0.f;
#pragma unroll
                    for (int q = 0; q < QD; ++q) {
                        const int u = lrd + LPRd * q;
                        const int uu = u < UI ? u : 0;
                        // this lane's unit of each row, decoded once; each h unit read once for all rows
                        u32 wd[RD][16];
                        float s0[RD], s1[RD];
#pragma unroll
                        for (int b = 0; b < RD; ++b) {
                            decode_unit<FMT, DEC>(un[st][b][q], Lt, wd[b]);
                            unit_scales<FMT>(un[st][b][q], Lt, s0[b], s1[b]);
                        }
#pragma unroll
                        for (int t = 0; t < XT; ++t) {
                            if (t < mb) {
                                const uint4 *hb = reinterpret_cast<const uint4 *>(s_buf + uu * USh + 32 * t);
                                u32 xh[16], xl[16];
#pragma unroll
                                for (int vv = 0; vv < 4; ++vv) {
                                    const uint4 A = hb[vv], B = hb[4 + vv];
                                    xh[4 * vv] = A.x; xh[4 * vv + 1] = A.y; xh[4 * vv + 2] = A.z; xh[4 * vv + 3] = A.w;
                                    xl[4 * vv] = B.x; xl[4 * vv + 1] = B.y; xl[4 * vv + 2] = B.z; xl[4 * vv + 3] = B.w;
                                }
#pragma unroll
                                for (int b = 0; b < RD; ++b) {
                                    const float d = unit_dot_split<FMT>(wd[b], xh, xl, s0[b], s1[b], acc[b][t]);
                                    acc[b][t] = u < UI ? d : acc[b][t];
                                }
                            }
                        }
                    }
#pragma unroll
                    for (int b = 0; b < RD; ++b) {
                        const int j = jrow(it, b);
#pragma unroll
                        for (int t = 0; t < XT; ++t) {
                            if (t < mb) {
                                const float ysum = group_sum_dpp(acc[b][t], LPRd);
                                if (j < nsub && lrd == 0)
                                    dt_store_tagged(yw, (u32)(o0 + j) * 8u, (u32)((pos0 + tb + t) * H) * 8u, tag, ysum);
                            }
                        }
                    }
                };
                // six-bit codes: one item per wave at a time (0.582 against 0.588 ms
                // for e2m3 + UE8M0, 0.617 against 0.626 for e2m3 + e4m3); four-bit
                // codes: two in flight (0.458 against 0.464 ms with one)
                if constexpr (Fmt<FMT>::SIX) {
                    for (;;) {
                        if (ia >= nitem) break;
                        compute(0, ia);
                        ia = grab();
                        issue(0, ia);
                    }
                } else {
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
                }
                ++nbatch;
            }
        }
    }

    // ------------------------------------------------ D. combine rows [w*RW, (w+1)*RW) of every token
    __syncthreads();
    {
        const int oo0 = w * plan.rw, nro = max(0, min(H, oo0 + plan.rw) - oo0);
        const int kk = k + (Ish > 0 ? 1 : 0);
        const __amdgpu_buffer_rsrc_t yr = rsrc_of(yq, (uint64_t)DEC_MAX_PAIRS * H * 8);
        for (int q = tid; q < T * nro; q += DT_THREADS) {
            const int t = q / nro, o = oo0 + (q - t * nro);
            // the token's partials in rank order, eight at a time (the shared expert last)
            float acc = 0.f;
            for (int r0 = 0; r0 < kk; r0 += 8) {
                float yv[8];
                u32 stale = 0;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int r = min(r0 + j, kk - 1);
                    const u32 off = (u32)(((size_t)S.pos_of[t][r] * H + o) * 8);
                    const uint2 v = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(yr, (int)off, 0, 0));
                    const u32 vx = v.x, vy = v.y;
                    yv[j] = __builtin_bit_cast(float, vx);
                    if (vy != tag) stale |= 1u << j;
                }
                while (stale != 0u) {
                    if (spins >= a.spin_limit) {
                        d1_st_relaxed(&hdr[WS_ERR], 1u);
                        break;
                    }
                    ++spins;
                    __builtin_amdgcn_s_sleep(1);
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        if (stale & (1u << j)) {
                            const int r = min(r0 + j, kk - 1);
                            const u32 off = (u32)(((size_t)S.pos_of[t][r] * H + o) * 8);
                            const uint2 v =
                                __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(yr, (int)off, 0, 16));   // sc1
                            const u32 vx = v.x, vy = v.y;
                            if (vy == tag) {
                                yv[j] = __builtin_bit_cast(float, vx);
                                stale &= ~(1u << j);
                            }
                        }
                    }
                }
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int r = r0 + j;
                    if (r < k) acc = __builtin_fmaf(S.w[t * k + r], yv[j], acc);
                    else if (r < kk) acc += yv[j];
                }
            }
            const int64_t oi = (int64_t)t * H + o;
            if (a.residual) acc += bf16_to_f32(a.residual[oi]);
            if (a.out_f32) reinterpret_cast<float *>(a.out)[oi] = acc;
            else reinterpret_cast<uint16_t *>(a.out)[oi] = f32_to_bf16_rne(acc);
        }
    }
    __syncthreads();
    if (tid == 0) __hip_atomic_fetch_max(&hdr[WS_EPOCH], tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int FMT, int DEC, int QG, int QD, int XT>
static hipError_t decodeT_launch(const DecodeArgs &a, hipStream_t s) {
    auto kern = decodeT_kernel<FMT, DEC, QG, QD, XT>;
    const LayerArgs &L = a.L;
    const int Imax = L.I > L.Ish ? L.I : L.Ish;
    int xt_gu = XT, xt_dn = XT;
    while (xt_gu > 0 && dt_lds_bytes(L.H / 32, 16, xt_gu) > DT_LDS) --xt_gu;
    // a batch's h fits LDS and one read pass (DT_HPT pieces per thread)
    while (xt_dn > 0 && (dt_lds_bytes(Imax / 32, 32, xt_dn) > DT_LDS ||
                         (size_t)xt_dn * (Imax / 2) > (size_t)DT_HPT * DT_THREADS))
        --xt_dn;
    if (xt_gu < 1 || xt_dn < 1) return hipErrorNotSupported;
    const size_t dyn = std::max(dt_lds_bytes(L.H / 32, 16, xt_gu), dt_lds_bytes(Imax / 32, 32, xt_dn));
    // dynamic LDS beyond the default limit (raised once per device)
    const hipError_t le = ensure_dyn_lds(reinterpret_cast<const void *>(kern), dyn);
    if (le != hipSuccess) return le;
    int cus = 0;
    const int cap = d1_coresident(kern, dyn, cus);
    const int G = std::min(cus, cap);   // every workgroup resident: they wait on each other
    if (G < 1) return hipErrorNotSupported;
    const DTPlan plan{G, (L.H + G - 1) / G, xt_gu, xt_dn};
    hipLaunchKernelGGL(kern, dim3(G), dim3(DT_THREADS), dyn, s, a, plan);
    return hipGetLastError();
}

template <int FMT, int DEC, int QG, int QD>
static hipError_t decodeT_go(const DecodeArgs &a, hipStream_t s) {
    if (a.L.Ish > 0 && a.T > 4) return decodeT_launch<FMT, DEC, QG, QD, 8>(a, s);
    return decodeT_launch<FMT, DEC, QG, QD, 4>(a, s);
}

template <int FMT, int DEC>
hipError_t decodeT_fd(const DecodeArgs &a, hipStream_t s) {
    const LayerArgs &L = a.L;
    if (a.T < 2 || a.T > DEC_MAX_T || a.mode != MODE_ROUTE || L.E > 1024 || L.k > 32) return hipErrorNotSupported;
    const int Imax = L.I > L.Ish ? L.I : L.Ish;
    const int UH = L.H / 32, QG = (UH + lanes_per_row(UH) - 1) / lanes_per_row(UH);
    const int LPRd = down_lanes_per_row(L.I, L.Ish), QD = (Imax / 32 + LPRd - 1) / LPRd;
    if (QG == 1 && QD == 1) return decodeT_go<FMT, DEC, 1, 1>(a, s);
    if (QG == 2 && QD == 1) return decodeT_go<FMT, DEC, 2, 1>(a, s);
    if (QG == 3 && QD == 1) return decodeT_go<FMT, DEC, 3, 1>(a, s);
    if (QG == 4 && QD == 1) return decodeT_go<FMT, DEC, 4, 1>(a, s);
    if (QG == 1 && QD == 2) return decodeT_go<FMT, DEC, 1, 2>(a, s);
    if (QG == 2 && QD == 2) return decodeT_go<FMT, DEC, 2, 2>(a, s);
    return hipErrorNotSupported;
}

}  // namespace moeq
