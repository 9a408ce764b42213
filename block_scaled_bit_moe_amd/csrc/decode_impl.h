// decode.hip -- the MoE layer for up to 16 tokens in one kernel launch.
//
// What it computes (Strata docs/INTEL.md, "The engine itself on Intel":
// router_top10, shared_expert; nextsycl README, "What it does": gate | up and
// down expert kernels, several rows decoded together with each row exactly as
// its own pass; colibri README, "DeepSeek V4": routed experts plus one shared):
//   route every token (top-k, softmax over the k picks),
//   group the (token, expert) pairs by expert (ascending expert id, tokens
//   ascending inside an expert),
//   per group: g, u = W13[e] x; h = silu(g) * u; y = W2[e] h,
//   out[t] = sum_r w[t][r] * y[pos(t, r)] + y_shared[t], in rank order.
//
// Shape of the launch: a persistent grid of G co-resident workgroups (G is
// capped by the occupancy the runtime reports, so every workgroup is resident
// at once).  Every workgroup routes all tokens and builds the work list in LDS
// itself -- a few microseconds of redundant work that avoids a second launch.
// Items are then taken round-robin in a fixed order:
//   gate/up items (group g, slice of DEC_S1 rows of I): write h as bf16 hi/lo;
//   down items (row slice j of H, group g), slice-major: write fp32 partials.
// A down item waits (bounded spin) until its group's gate/up items are done;
// all gate/up items precede all down items in every workgroup's sequence, so
// the oldest unfinished item never waits.  The last workgroup to finish a row
// slice (atomic ticket) sums that slice's partials in rank order and stores
// the output; no float atomics touch the output, so results are bitwise
// reproducible and independent of which tokens share the call.
// Every spin is bounded (Strata docs/INTEL.md, "The engine itself on Intel":
// an unbounded device spin wedges the card); on expiry the kernel sets the
// workspace error word and runs to completion.  The last workgroup to exit
// returns every counter to zero.
#pragma once

#include "kernels.h"
#include "rowdot.h"

namespace moeq {

// Inter-workgroup traffic.  Data that one workgroup writes and another reads
// inside the launch (h and the fp32 partials) moves with device-coherent
// (sc1) stores and loads, so no L2 write-back or invalidate is ever needed;
// a writer waits for its stores to complete (s_waitcnt vmcnt(0)) before it
// bumps a relaxed counter, and a reader issues its loads only after it has
// seen the count.
__device__ inline u32 ld_relaxed_agent(const u32 *p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ inline void st_relaxed_agent(u32 *p, u32 v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ inline u32 add_relaxed_agent(u32 *p, u32 v) { return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ inline void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

typedef __attribute__((ext_vector_type(4))) u32 u32x4_t;
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, u32 bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
// 16 bytes at byte offset `off`, read at device coherence (sc1)
__device__ inline u32x4_t ld16_coherent(__amdgpu_buffer_rsrc_t r, u32 off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 16);
}

// h of one (token, expert) pair is stored as 32-bit words, unit by unit: the
// 32 elements of unit u occupy words [32u, 32u+32): first 16 words hold the
// bf16 "hi" parts of element pairs (2i, 2i+1), the next 16 the "lo" parts
// (h = hi + lo to about 16 significant bits).
template <int Q, int MT>
__device__ inline void load_h_units(u32 (&xh)[Q][MT][16], u32 (&xl)[Q][MT][16], __amdgpu_buffer_rsrc_t r,
                                    const int (&pos)[MT], int Imax, int U, int lr, int LPR) {
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int u = lr + LPR * q;
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            if (u < U && pos[t] >= 0) {
                const u32 base = (u32)((pos[t] * Imax + 32 * u) * 4);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    u32x4_t a = ld16_coherent(r, base + 16 * v);
                    xh[q][t][4 * v + 0] = a.x; xh[q][t][4 * v + 1] = a.y; xh[q][t][4 * v + 2] = a.z; xh[q][t][4 * v + 3] = a.w;
                    u32x4_t b = ld16_coherent(r, base + 64 + 16 * v);
                    xl[q][t][4 * v + 0] = b.x; xl[q][t][4 * v + 1] = b.y; xl[q][t][4 * v + 2] = b.z; xl[q][t][4 * v + 3] = b.w;
                }
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i) { xh[q][t][i] = 0u; xl[q][t][i] = 0u; }
            }
        }
    }
}

template <int MT>
struct DecShared {
    int idx[DEC_MAX_T * 32];
    float w[DEC_MAX_T * 32];
    u32 mask[1024];
    short e2g[1024];
    short g_expert[DEC_MAX_GROUPS];   // -1: the shared expert
    short g_start[DEC_MAX_GROUPS];
    short g_count[DEC_MAX_GROUPS];
    unsigned char p_tok[DEC_MAX_PAIRS];
    short pos_of[DEC_MAX_T][33];
    int scan[16];
    int n_groups, n_pairs, n_routed_groups, kk, flag;
    float gu[2 * DEC_S1][MT];
};

// exclusive block scan of two counters (blockDim.x == 256)
__device__ inline void block_exscan2(int a, int b, int &ea, int &eb, int &ta, int &tb, int *tmp) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int ia = a, ib = b;
    for (int m = 1; m < 64; m <<= 1) {
        int oa = __shfl_up(ia, m, WAVE), ob = __shfl_up(ib, m, WAVE);
        if (lane >= m) { ia += oa; ib += ob; }
    }
    if (lane == 63) { tmp[wv] = ia; tmp[4 + wv] = ib; }
    __syncthreads();
    int pa = 0, pb = 0;
    for (int v = 0; v < wv; ++v) { pa += tmp[v]; pb += tmp[4 + v]; }
    ta = tmp[0] + tmp[1] + tmp[2] + tmp[3];
    tb = tmp[4] + tmp[5] + tmp[6] + tmp[7];
    ea = pa + ia - a;
    eb = pb + ib - b;
    __syncthreads();
}

template <int PL>
__device__ inline void route_tokens(const DecodeArgs &a, int T, int E, int k, int *s_idx, float *s_w) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    for (int t = wv; t < T; t += 4) {
        int e;
        float wt;
        route_one_token_wave<PL>(a.logits + (int64_t)t * E, E, k, lane, e, wt);
        if (lane < k) {
            s_idx[t * k + lane] = e;
            s_w[t * k + lane] = wt;
            if (blockIdx.x == 0) {
                if (a.idx_out) a.idx_out[(int64_t)t * k + lane] = e;
                if (a.w_out) a.w_out[(int64_t)t * k + lane] = wt;
            }
        }
    }
}

template <int FMT, int DEC, int QG, int QD, int MT>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
    constexpr int PAIR = (DEC == DEC_LUT) ? (Fmt<FMT>::SIX ? LUT_E2M3_PAIR : LUT_E2M1_PAIR) : 1;
    __shared__ u32 s_pair[PAIR];
    __shared__ float s_scale[LUT_SCALE];
    __shared__ DecShared<MT> S;
    const Luts L{s_pair, s_scale};
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const LayerArgs &ly = a.L;
    const int T = a.T, H = ly.H, I = ly.I, E = ly.E, Ish = ly.Ish;
    const int Imax = I > Ish ? I : Ish;
    u32 *hdr = reinterpret_cast<u32 *>(a.ws);
    u32 *hl = reinterpret_cast<u32 *>(a.ws + WS_HEADER);                 // [pairs][Imax] words
    u32 *ybuf = hl + (size_t)DEC_MAX_PAIRS * Imax;                         // [pairs][H] fp32 bits
    const __amdgpu_buffer_rsrc_t hl_rsrc = make_rsrc(hl, (u32)((size_t)DEC_MAX_PAIRS * Imax * 4));

    build_luts<FMT>(L, tid, 256, DEC == DEC_LUT);

    // ---------------------------------------------------------- route + work list
    if (a.mode == MODE_ROUTE) {
        const int k = ly.k;
        if (E <= 64) route_tokens<1>(a, T, E, k, S.idx, S.w);
        else if (E <= 128) route_tokens<2>(a, T, E, k, S.idx, S.w);
        else if (E <= 256) route_tokens<4>(a, T, E, k, S.idx, S.w);
        else if (E <= 512) route_tokens<8>(a, T, E, k, S.idx, S.w);
        else route_tokens<16>(a, T, E, k, S.idx, S.w);
        for (int e = tid; e < 1024; e += 256) S.mask[e] = 0u;
        __syncthreads();
        for (int p = tid; p < T * k; p += 256) atomicOr(&S.mask[S.idx[p]], 1u << (p / k));
        __syncthreads();
        // scan over experts: group index and first pair position of each used expert
        const int e0 = tid * 4;
        int f[4], c[4], tf = 0, tc = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            u32 m = (e0 + j < E) ? S.mask[e0 + j] : 0u;
            f[j] = m != 0u;
            c[j] = __builtin_popcount(m);
            tf += f[j];
            tc += c[j];
        }
        int ef, ec, nf, nc;
        block_exscan2(tf, tc, ef, ec, nf, nc, S.scan);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (f[j]) {
                const int e = e0 + j;
                S.e2g[e] = (short)ef;
                S.g_expert[ef] = (short)e;
                S.g_start[ef] = (short)ec;
                S.g_count[ef] = (short)c[j];
                u32 m = S.mask[e];
                int n = 0;
                while (m) {
                    int t = __builtin_ctz(m);
                    m &= m - 1u;
                    S.p_tok[ec + n++] = (unsigned char)t;
                }
                ef += 1;
                ec += c[j];
            }
        }
        __syncthreads();
        for (int p = tid; p < T * k; p += 256) {
            const int t = p / k, r = p % k, e = S.idx[p];
            const int g = S.e2g[e];
            S.pos_of[t][r] = (short)(S.g_start[g] + __builtin_popcount(S.mask[e] & ((1u << t) - 1u)));
        }
        if (tid == 0) {
            S.n_routed_groups = nf;
            S.n_groups = nf;
            S.n_pairs = nc;
            S.kk = k;
            if (Ish > 0) {
                S.g_expert[nf] = -1;
                S.g_start[nf] = (short)nc;
                S.g_count[nf] = (short)T;
                S.n_groups = nf + 1;
                S.n_pairs = nc + T;
            }
        }
        __syncthreads();
        if (Ish > 0)
            for (int t = tid; t < T; t += 256) {
                S.p_tok[S.g_start[S.n_routed_groups] + t] = (unsigned char)t;
                S.pos_of[t][k] = (short)(S.g_start[S.n_routed_groups] + t);
            }
    } else {
        // one expert applied to all T rows, weight 1
        if (tid == 0) {
            const bool sh = (a.mode == MODE_FIXED_SHARED);
            S.g_expert[0] = sh ? -1 : (short)a.fixed_e;
            S.g_start[0] = 0;
            S.g_count[0] = (short)T;
            S.n_groups = 1;
            S.n_routed_groups = sh ? 0 : 1;
            S.n_pairs = T;
            S.kk = 1;
        }
        for (int t = tid; t < T; t += 256) {
            S.p_tok[t] = (unsigned char)t;
            S.pos_of[t][0] = (short)t;
            S.w[t] = 1.0f;
        }
    }
    __syncthreads();

    // ---------------------------------------------------------- items
    const int NG = S.n_groups, NRG = S.n_routed_groups, kk = S.kk;
    const bool add_shared = (a.mode == MODE_ROUTE) && (Ish > 0);
    const int64_t crbH = Fmt<FMT>::code_row_bytes(H), srbH = Fmt<FMT>::scale_row_bytes(H);
    const int UH = H / 32, LPRg = lanes_per_row(UH), RPWg = WAVE / LPRg;
    const int lrg = lane & (LPRg - 1), rsg = lane / LPRg;
    constexpr int S1 = DEC_S1;
    const int gu_per_routed = I / S1, gu_shared = Ish / S1;
    const int n_gu = NRG * gu_per_routed + (NG - NRG) * gu_shared;
    const int n_slices = (H + DEC_S2 - 1) / DEC_S2;
    const int total = n_gu + n_slices * NG;
    u32 *gu_done = hdr + WS_GU, *dn_done = hdr + WS_DN;

    for (int item = blockIdx.x; item < total; item += gridDim.x) {
        if (item < n_gu) {
            // ------------------------------------------------ gate | up, SiLU-multiply
            int g, s;
            if (item < NRG * gu_per_routed) { g = item / gu_per_routed; s = item % gu_per_routed; }
            else { g = NRG; s = item - NRG * gu_per_routed; }
            const int e = S.g_expert[g];
            const int Ig = (e >= 0) ? I : Ish;
            const uint8_t *c13 = (e >= 0) ? ly.w13c + (int64_t)e * 2 * I * crbH : ly.sh13c;
            const uint8_t *s13 = (e >= 0) ? ly.w13s + (int64_t)e * 2 * I * srbH : ly.sh13s;
            const int mg = S.g_count[g], pos0 = S.g_start[g];
            for (int tt = 0; tt < mg; tt += MT) {
                u32 xr[QG][MT][16];
                const uint16_t *xp[MT];
#pragma unroll
                for (int j = 0; j < MT; ++j)
                    xp[j] = (tt + j < mg) ? a.x + (int64_t)S.p_tok[pos0 + tt + j] * H : nullptr;
                load_x_units<QG, MT>(xr, xp, UH, lrg, LPRg);
                // rows v of the item (gate rows 0..S1-1, up rows S1..2*S1-1), streamed R per pass
                constexpr int R = 2;
                const int npass = (2 * S1 + 4 * RPWg * R - 1) / (4 * RPWg * R);
                auto row = [&](int p, int b, const uint8_t *&c, const uint8_t *&sc) -> int {
                    const int v = p * 4 * RPWg * R + wv * RPWg + b * 4 * RPWg + rsg;
                    const int vv = v < 2 * S1 ? v : 0;
                    const int r = vv < S1 ? s * S1 + vv : Ig + s * S1 + (vv - S1);
                    c = c13 + (int64_t)r * crbH;
                    sc = s13 + (int64_t)r * srbH;
                    return v < 2 * S1 ? v : -1;
                };
                auto out = [&](int, int, int v, const float (&acc)[MT]) {
                    if (v >= 0 && lrg == 0)
#pragma unroll
                        for (int j = 0; j < MT; ++j) S.gu[v][j] = acc[j];
                };
                RowPipe<FMT, DEC, QG, MT, R, false> pipe;
                pipe.begin(row, UH, lrg, LPRg);
                pipe.run(npass, row, UH, lrg, LPRg, xr, xr, L, out);
                __syncthreads();
                for (int q = tid; q < (S1 / 2) * MT; q += 256) {
                    const int kp = q / MT, j = q % MT;
                    if (tt + j < mg) {
                        const int i0 = 2 * kp;
                        const float h0 = silu_f32(S.gu[i0][j]) * S.gu[S1 + i0][j];
                        const float h1 = silu_f32(S.gu[i0 + 1][j]) * S.gu[S1 + i0 + 1][j];
                        const u32 hi0 = f32_to_bf16_rne(h0), hi1 = f32_to_bf16_rne(h1);
                        const u32 lo0 = f32_to_bf16_rne(h0 - __builtin_bit_cast(float, hi0 << 16));
                        const u32 lo1 = f32_to_bf16_rne(h1 - __builtin_bit_cast(float, hi1 << 16));
                        const int p = (s * S1 + i0) >> 1, uu = p >> 4, kk2 = p & 15;
                        u32 *row = hl + (size_t)(pos0 + tt + j) * Imax + 32 * uu;
                        st_relaxed_agent(row + kk2, hi0 | (hi1 << 16));
                        st_relaxed_agent(row + 16 + kk2, lo0 | (lo1 << 16));
                    }
                }
                __syncthreads();
            }
            wait_stores();
            __syncthreads();
            if (tid == 0) add_relaxed_agent(&gu_done[g], 1u);
        } else {
            // ------------------------------------------------ down projection partials
            const int d = item - n_gu;
            const int j = d / NG, g = d % NG;
            const int e = S.g_expert[g];
            const int Ig = (e >= 0) ? I : Ish;
            const u32 need = (u32)(Ig / S1);
            const int64_t crbI = Fmt<FMT>::code_row_bytes(Ig), srbI = Fmt<FMT>::scale_row_bytes(Ig);
            const uint8_t *c2 = (e >= 0) ? ly.w2c + (int64_t)e * H * crbI : ly.sh2c;
            const uint8_t *s2 = (e >= 0) ? ly.w2s + (int64_t)e * H * srbI : ly.sh2s;
            const int UI = Ig / 32, LPRd = down_lanes_per_row(I, Ish), RPWd = WAVE / LPRd;
            const int lrd = lane & (LPRd - 1), rsd = lane / LPRd;
            const int mg = S.g_count[g], pos0 = S.g_start[g];
            const int o_lo = j * DEC_S2, o_hi = (o_lo + DEC_S2 < H) ? o_lo + DEC_S2 : H;
            // output rows o of the slice, streamed R per pass
            constexpr int R = 2;
            const int npass = (o_hi - o_lo + 4 * RPWd * R - 1) / (4 * RPWd * R);
            auto row = [&](int p, int b, const uint8_t *&c, const uint8_t *&sc) -> int {
                const int o = o_lo + p * 4 * RPWd * R + wv * RPWd + b * 4 * RPWd + rsd;
                const int oo = o < o_hi ? o : o_lo;
                c = c2 + (int64_t)oo * crbI;
                sc = s2 + (int64_t)oo * srbI;
                return o < o_hi ? o : -1;
            };
            RowPipe<FMT, DEC, QD, MT, R, true> pipe;
            pipe.begin(row, UI, lrd, LPRd);   // the weights do not depend on h: in flight during the wait
            if (tid == 0) {
                // bounded wait; spin_limit 0 (the test hook) expires at once without polling
                u32 spins = 0;
                while (a.spin_limit == 0u || ld_relaxed_agent(&gu_done[g]) < need) {
                    if (spins++ >= a.spin_limit) { st_relaxed_agent(&hdr[WS_ERR], 1u); break; }
                    __builtin_amdgcn_s_sleep(2);
                }
            }
            __syncthreads();
            for (int tt = 0; tt < mg; tt += MT) {
                u32 xh[QD][MT][16], xl[QD][MT][16];
                int pp[MT];
#pragma unroll
                for (int jj = 0; jj < MT; ++jj) pp[jj] = (tt + jj < mg) ? pos0 + tt + jj : -1;
                load_h_units<QD, MT>(xh, xl, hl_rsrc, pp, Imax, UI, lrd, LPRd);
                auto out = [&](int, int, int o, const float (&acc)[MT]) {
                    if (o >= 0 && lrd == 0)
#pragma unroll
                        for (int jj = 0; jj < MT; ++jj)
                            if (tt + jj < mg)
                                st_relaxed_agent(ybuf + (size_t)(pos0 + tt + jj) * H + o, __builtin_bit_cast(u32, acc[jj]));
                };
                if (tt > 0) pipe.begin(row, UI, lrd, LPRd);
                pipe.run(npass, row, UI, lrd, LPRd, xh, xl, L, out);
            }
            wait_stores();
            __syncthreads();
            if (tid == 0) S.flag = (add_relaxed_agent(&dn_done[j], 1u) == (u32)(NG - 1));
            __syncthreads();
            if (S.flag) {
                // ------------------------------------------------ combine this row slice
                const int width = o_hi - o_lo;
                for (int q = tid; q < T * width; q += 256) {
                    const int t = q / width, o = o_lo + q % width;
                    float acc = 0.f;
                    for (int r = 0; r < kk; ++r)
                        acc = __builtin_fmaf(S.w[t * kk + r],
                                             __builtin_bit_cast(float, ld_relaxed_agent(ybuf + (size_t)S.pos_of[t][r] * H + o)),
                                             acc);
                    if (add_shared) acc += __builtin_bit_cast(float, ld_relaxed_agent(ybuf + (size_t)S.pos_of[t][kk] * H + o));
                    const int64_t oi = (int64_t)t * H + o;
                    if (a.residual) acc += bf16_to_f32(a.residual[oi]);
                    if (a.out_f32) reinterpret_cast<float *>(a.out)[oi] = acc;
                    else reinterpret_cast<uint16_t *>(a.out)[oi] = f32_to_bf16_rne(acc);
                }
            }
            __syncthreads();
        }
    }

    // ---------------------------------------------------------- exit: the last workgroup resets
    wait_stores();
    __syncthreads();
    if (tid == 0) {
        const u32 old = add_relaxed_agent(&hdr[WS_EXIT], 1u);
        if (old == gridDim.x - 1) {
            for (int g = 0; g < NG; ++g) st_relaxed_agent(&gu_done[g], 0u);
            for (int j = 0; j < n_slices; ++j) st_relaxed_agent(&dn_done[j], 0u);
            st_relaxed_agent(&hdr[WS_EXIT], 0u);
        }
    }
}

// ---------------------------------------------------------------- launch
// Workgroups of `kernel` resident at once on the current device (cached).
template <typename K>
static int coresident_blocks(K kernel) {
    const int per = cached_occupancy(reinterpret_cast<const void *>(kernel), 256, 0);
    return (per > 0 ? per : 1) * cached_cus();
}

template <int FMT, int DEC, int QG, int QD, int MT>
static hipError_t decode_go(const DecodeArgs &a, hipStream_t s) {
    auto kern = decode_kernel<FMT, DEC, QG, QD, MT>;
    const int cap = coresident_blocks(kern);
    // upper bound of the item count: every pair its own group
    const LayerArgs &L = a.L;
    const int groups = (a.mode == MODE_ROUTE) ? ((a.T * L.k < L.E ? a.T * L.k : L.E) + (L.Ish > 0)) : 1;
    const int n_gu = groups * ((L.I > L.Ish ? L.I : L.Ish) / DEC_S1);
    const int n_dn = ((L.H + DEC_S2 - 1) / DEC_S2) * groups;
    int G = n_gu + n_dn;
    if (G > cap) G = cap;
    hipLaunchKernelGGL(kern, dim3(G), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int FMT, int DEC, int QG>
static hipError_t decode_qd(const DecodeArgs &a, int QD, int MT, hipStream_t s) {
#define GO(QQ)                                                       \
    if (QD == QQ) {                                                  \
        if (MT == 1) return decode_go<FMT, DEC, QG, QQ, 1>(a, s);   \
        return decode_go<FMT, DEC, QG, QQ, 2>(a, s);                \
    }
    GO(1) GO(2) GO(3) GO(4)
#undef GO
    return hipErrorInvalidValue;
}

template <int FMT, int DEC>
hipError_t decode_fd(const DecodeArgs &a, hipStream_t s) {
    const LayerArgs &L = a.L;
    const int UH = L.H / 32, QG = (UH + lanes_per_row(UH) - 1) / lanes_per_row(UH);
    const int Imax = L.I > L.Ish ? L.I : L.Ish;
    // QD must cover both the routed and the shared intermediate size
    const int LPRd = down_lanes_per_row(L.I, L.Ish);
    const int QD = ((Imax / 32) + LPRd - 1) / LPRd;
    (void)Imax;
    const int MT = (a.T == 1) ? 1 : 2;
    switch (QG) {
        case 1: return decode_qd<FMT, DEC, 1>(a, QD, MT, s);
        case 2: return decode_qd<FMT, DEC, 2>(a, QD, MT, s);
        case 3: return decode_qd<FMT, DEC, 3>(a, QD, MT, s);
        case 4: return decode_qd<FMT, DEC, 4>(a, QD, MT, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace moeq
